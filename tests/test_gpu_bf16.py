"""GPU parity of mha_fwd_bf16 against the float64 oracle (needs an MI355X)."""

import numpy as np
import pytest
import torch

import workloads
from parity import (assert_bf16_parity, assert_every_block_row, oracle_heads, require_gpu, scale_for, to_np)

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal, scale=None):
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = mha.mha_fwd_bf16(qd, kd, vd, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check_all(q, k, v, causal, what, scale=None):
    b, sq, hq, dqk = q.shape
    scale = scale_for(dqk) if scale is None else scale
    o, lse = _run(q, k, v, causal, scale)
    for bb in range(b):
        o_ref, l_ref = oracle_heads(q, k, v, list(range(hq)), None, scale=scale, causal=causal, batch=bb)
        assert_bf16_parity(to_np(o[bb]), o_ref, lse[bb].numpy().astype(np.float64), l_ref, f"{what} b={bb}")


def test_tiny_d64_full():
    w = workloads.WORKLOADS["tiny_d64"]
    q, k, v = workloads.make_qkv(w)
    _check_all(q, k, v, w.causal, "tiny_d64")


SMALL_SHAPES = [
    # b, hq, hk, sq, sk, dqk, dv
    (2, 4, 2, 300, 300, 64, 64),
    (1, 6, 1, 257, 257, 64, 64),
    (1, 4, 4, 200, 333, 128, 128),
    (2, 2, 1, 333, 200, 128, 128),
    (1, 2, 2, 190, 190, 192, 128),
    (1, 3, 3, 129, 65, 192, 128),
    # several 256-row blocks: causal pairs whose light block runs its tiles downward, with a
    # ragged last block, more keys than queries and fewer
    (1, 2, 2, 700, 700, 192, 128),
    (1, 2, 1, 600, 800, 192, 128),
    (2, 2, 2, 800, 520, 192, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=[f"b{s[0]}h{s[1]}/{s[2]}q{s[3]}k{s[4]}d{s[5]}-{s[6]}" for s in SMALL_SHAPES])
def test_multi_tile_ragged(shape, causal):
    b, hq, hk, sq, sk, dqk, dv = shape
    seed = 1000 + sum(shape) + int(causal)
    q = workloads.make_random((b, sq, hq, dqk), seed)
    k = workloads.make_random((b, sk, hk, dqk), seed + 1)
    v = workloads.make_random((b, sk, hk, dv), seed + 2)
    _check_all(q, k, v, causal, f"shape={shape} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq, sk", [(200, 200), (200, 333), (300, 160)])
def test_two_heads_per_workgroup(sq, sk, causal):
    # d128 GQA grids that still fill the device with two query heads per workgroup (hq 512 over
    # hk 256: 256 workgroups of 8 waves) take the packed kernel: waves 0-3 of a workgroup serve
    # head 2i, waves 4-7 head 2i+1, on the same K/V tiles.  Ragged blocks, more and fewer keys
    # than queries.
    q = workloads.make_random((1, sq, 512, 128), 4300 + sq + int(causal))
    k = workloads.make_random((1, sk, 256, 128), 4301 + sk)
    v = workloads.make_random((1, sk, 256, 128), 4302 + sk)
    o, lse = _run(q, k, v, causal)
    heads = list(range(0, 512, 37)) + [1, 2, 3, 510, 511]
    o_ref, l_ref = oracle_heads(q, k, v, heads, None, scale=scale_for(128), causal=causal, batch=0)
    assert_bf16_parity(to_np(o[0][:, heads]), o_ref, lse[0][heads].numpy().astype(np.float64), l_ref,
                       f"two heads per workgroup {sq}x{sk} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_two_heads_per_workgroup_batched(causal):
    # the packed kernel over two batches (hq 256 over hk 128: 256 workgroups), every batch checked
    q = workloads.make_random((2, 200, 256, 128), 4400 + int(causal))
    k = workloads.make_random((2, 260, 128, 128), 4401)
    v = workloads.make_random((2, 260, 128, 128), 4402)
    o, lse = _run(q, k, v, causal)
    heads = list(range(0, 256, 29)) + [1, 254, 255]
    for bb in range(2):
        o_ref, l_ref = oracle_heads(q, k, v, heads, None, scale=scale_for(128), causal=causal, batch=bb)
        assert_bf16_parity(to_np(o[bb][:, heads]), o_ref, lse[bb][heads].numpy().astype(np.float64), l_ref,
                           f"two heads per workgroup b={bb} causal={causal}")


def _full_size_sampled(name, heads, nrows, seed):
    """The full-size launch: many seeded rows (and the block edges) of a few heads, plus one
    seeded row of every (batch, head, 128-row block), i.e. of every workgroup."""
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_qkv(w)
    o, lse = _run(q, k, v, w.causal, w.scale)
    rows = workloads.sample_indices(w.sq, nrows, seed, include=[0, 1, 63, 64, 127, 128, w.sq // 2, w.sq - 1])
    batches = sorted({0, w.b - 1})
    for bb in batches:
        o_ref, l_ref = oracle_heads(q, k, v, heads, rows, scale=w.scale, causal=w.causal, batch=bb)
        o_g = to_np(o[bb][rows][:, heads])
        l_g = lse[bb][heads][:, rows].numpy().astype(np.float64)
        assert_bf16_parity(o_g, o_ref, l_g, l_ref, f"{name} b={bb} heads={heads}")
    assert_every_block_row(q, k, v, o, lse, scale=w.scale, causal=w.causal, seed=seed, what=name)


def test_full_gqa_d64_causal_sampled():
    # two query heads that share kv head 0, one from each other group edge
    _full_size_sampled("gqa_d64_causal", [0, 1, 5, 6, 23, 47], 192, 7)


def test_full_gqa_d128_causal_sampled():
    _full_size_sampled("gqa_d128_causal", [0, 3, 4, 31], 192, 8)


def test_full_mla_d192_d128_causal_sampled():
    _full_size_sampled("mla_d192_d128_causal", [0, 77, 127], 160, 9)


def test_full_mla_d192_d128_noncausal_sampled():
    _full_size_sampled("mla_d192_d128_noncausal", [0, 64, 127], 128, 10)


def test_full_gqa_d128_8192_causal_sampled():
    # heads 15 and 16 sit on either side of a kv-head boundary (16 query heads per kv head)
    _full_size_sampled("gqa_d128_8192_causal", [0, 15, 16, 127], 128, 11)


def test_full_mla_tp8_causal_sampled():
    _full_size_sampled("mla_d192_d128_tp8_causal", [0, 15], 160, 12)


def test_full_gqa8_d128_tp8_noncausal_sampled():
    # one rank's share of 8-way head sharding of a 64-query-head, 8-kv-head model: 8 query heads
    # on one kv head (GQA 8:1)
    _full_size_sampled("gqa8_d128_tp8_noncausal", [0, 3, 7], 128, 13)


def test_full_gqa5_d128_tp8_noncausal_sampled():
    # 40 query heads over 8 kv heads, one rank of 8: 5 query heads on one kv head (GQA 5:1)
    _full_size_sampled("gqa5_d128_tp8_noncausal", [0, 2, 4], 128, 14)


def test_full_gqa8_d128_tp8_causal_sampled():
    # the same rank's causal prefill: 256 causal pairs, one workgroup per CU (unsplit)
    _full_size_sampled("gqa8_d128_tp8_causal", [0, 5, 7], 128, 15)


def test_full_gqa5_d128_tp8_causal_sampled():
    # GQA 5:1 causal: 160 pairs, which the default call divides by key range (pairs of blocks
    # whose ranges cross from one block into the other)
    _full_size_sampled("gqa5_d128_tp8_causal", [0, 2, 4], 128, 16)


def test_value_ones_gives_ones():
    # V = 1 everywhere: every output row is 1 whatever the scores, up to the bf16 rounding of
    # the probabilities fed to the P.V product and of O itself.
    dev = require_gpu()
    import head_attention_forward_flash_amd as mha
    q = workloads.make_random((1, 300, 4, 128), 11, std=3.0).to(dev)
    k = workloads.make_random((1, 300, 2, 128), 12, std=3.0).to(dev)
    v = torch.ones((1, 300, 2, 128), dtype=torch.bfloat16, device=dev)
    for causal in (False, True):
        o, _ = mha.mha_fwd_bf16(q, k, v, causal=causal)
        assert torch.all((o.float() - 1.0).abs() <= 2.0 ** -7)


def test_causal_row_zero_equals_v0():
    dev = require_gpu()
    import head_attention_forward_flash_amd as mha
    q = workloads.make_random((2, 130, 6, 64), 21).to(dev)
    k = workloads.make_random((2, 130, 2, 64), 22).to(dev)
    v = workloads.make_random((2, 130, 2, 64), 23).to(dev)
    o, lse = mha.mha_fwd_bf16(q, k, v, causal=True)
    for h in range(6):
        assert torch.equal(o[:, 0, h, :], v[:, 0, h // 3, :])
    s00 = (q[:, 0].float() * k[:, 0].float().repeat_interleave(3, dim=1)).sum(-1) * 0.125
    assert torch.allclose(lse[:, :, 0], s00, atol=1e-4, rtol=0)


def test_strided_views_match_contiguous():
    # Q/K/V as slices of one packed [b, s, 3, h, d] tensor, O written into a wider buffer.
    dev = require_gpu()
    import head_attention_forward_flash_amd as mha
    qkv = workloads.make_random((2, 200, 3, 4, 128), 31).to(dev)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    big = torch.zeros((2, 200, 6, 128), dtype=torch.bfloat16, device=dev)
    out = big[:, :, 1:5]
    for causal in (False, True):
        o1, l1 = mha.mha_fwd_bf16(q, k, v, causal=causal, out=out)
        o2, l2 = mha.mha_fwd_bf16(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.all(big[:, :, 0] == 0) and torch.all(big[:, :, 5] == 0)


def test_deterministic():
    dev = require_gpu()
    import head_attention_forward_flash_amd as mha
    q = workloads.make_random((1, 1000, 8, 128), 41).to(dev)
    k = workloads.make_random((1, 1000, 2, 128), 42).to(dev)
    v = workloads.make_random((1, 1000, 2, 128), 43).to(dev)
    a = mha.mha_fwd_bf16(q, k, v, causal=True)
    b = mha.mha_fwd_bf16(q, k, v, causal=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_degenerate_sizes():
    dev = require_gpu()
    import head_attention_forward_flash_amd as mha
    # no keys: O = 0, LSE = -inf
    q = workloads.make_random((1, 5, 2, 64), 51).to(dev)
    k = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device=dev)
    v = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device=dev)
    o, lse = mha.mha_fwd_bf16(q, k, v, causal=False)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # no queries / no batch: no-ops
    q0 = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device=dev)
    k1 = workloads.make_random((1, 7, 2, 64), 52).to(dev)
    o, lse = mha.mha_fwd_bf16(q0, k1, k1, causal=True)
    assert o.shape == (1, 0, 2, 64)
    qb = torch.empty((0, 4, 2, 64), dtype=torch.bfloat16, device=dev)
    kb = torch.empty((0, 4, 2, 64), dtype=torch.bfloat16, device=dev)
    o, lse = mha.mha_fwd_bf16(qb, kb, kb)
    assert o.shape == (0, 4, 2, 64)
    # one query, one key
    q = workloads.make_random((1, 1, 1, 192), 53)
    k = workloads.make_random((1, 1, 1, 192), 54)
    v = workloads.make_random((1, 1, 1, 128), 55)
    o, lse = _run(q, k, v, True)
    assert torch.equal(o[0, 0, 0], v[0, 0, 0])
    _check_all(q, k, v, False, "1x1")


def test_large_score_magnitudes():
    # scores of magnitude ~100: exercises the running-max updates
    q = workloads.make_random((1, 256, 2, 64), 61, std=4.0)
    k = workloads.make_random((1, 256, 2, 64), 62, std=4.0)
    v = workloads.make_random((1, 256, 2, 64), 63)
    _check_all(q, k, v, False, "large scores", scale=0.5)
    _check_all(q, k, v, True, "large scores causal", scale=0.5)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
def test_negative_and_zero_scale(dims):
    # A negative scale flips the score order (the kernel negates Q, which is exact); a zero
    # scale makes every unmasked key equally likely, so O is the running mean of V and the
    # LSE is log(number of unmasked keys).  Both against the oracle, causal and not.
    dqk, dv = dims
    seed = 3000 + dqk
    q = workloads.make_random((1, 150, 2, dqk), seed)
    k = workloads.make_random((1, 150, 2, dqk), seed + 1)
    v = workloads.make_random((1, 150, 2, dv), seed + 2)
    for causal in (False, True):
        _check_all(q, k, v, causal, f"d{dqk} scale=-0.3 causal={causal}", scale=-0.3)
        _check_all(q, k, v, causal, f"d{dqk} scale=0 causal={causal}", scale=0.0)
    o, lse = _run(q, k, v, True, 0.0)
    counts = np.arange(1, 151, dtype=np.float64)
    np.testing.assert_allclose(lse[0, 0].numpy(), np.log(counts), atol=2 ** -8)


def test_negative_scale_in_pairs():
    # The sign flip of a negative scale runs in every block's prologue: both blocks of a causal
    # pair (d192: 700 rows are 3 blocks of 256, the pair (2, 0) and the middle block 1) and the
    # two-heads-per-workgroup kernel's pairs (hq 512 over hk 256, 3 blocks of 128).
    q = workloads.make_random((1, 700, 2, 192), 3400)
    k = workloads.make_random((1, 700, 2, 192), 3401)
    v = workloads.make_random((1, 700, 2, 128), 3402)
    _check_all(q, k, v, True, "d192 scale=-0.2 causal pairs", scale=-0.2)
    q = workloads.make_random((1, 300, 512, 128), 3403)
    k = workloads.make_random((1, 300, 256, 128), 3404)
    v = workloads.make_random((1, 300, 256, 128), 3405)
    o, lse = _run(q, k, v, True, -0.15)
    heads = list(range(0, 512, 41)) + [1, 510, 511]
    o_ref, l_ref = oracle_heads(q, k, v, heads, None, scale=-0.15, causal=True, batch=0)
    assert_bf16_parity(to_np(o[0][:, heads]), o_ref, lse[0][heads].numpy().astype(np.float64), l_ref,
                       "two heads per workgroup scale=-0.15 causal pairs")

def _ramp_inputs(dqk, dv, s, step, seed, rising):
    # every query points along channel 0 and key j carries step * j there (reversed when not
    # rising), so each row's scores climb (or fall) steadily along the keys; the other channels
    # hold small noise
    q = workloads.make_random((1, s, 2, dqk), seed, dtype=torch.float32, std=0.05)
    k = workloads.make_random((1, s, 2, dqk), seed + 1, dtype=torch.float32, std=0.05)
    q[..., 0] = 1.0
    j = torch.arange(s, dtype=torch.float32)
    k[0, :, :, 0] = (step * (j if rising else s - 1 - j))[:, None]
    v = workloads.make_random((1, s, 2, dv), seed + 2)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
def test_running_max_rising_in_steps(dims):
    # With a key step of 2^-4, the row max moves by 32 * 2^-4 * scale * log2(e) per 32-key block:
    # about 2 (scale 0.7, below the 2^8 rescale threshold, so the reference max lags and P
    # reaches up to 2^8 before a rescale) or about 29 (scale 10, a rescale every block).  Falling
    # scores fix the max on the first block instead.
    dqk, dv = dims
    for rising in (True, False):
        q, k, v = _ramp_inputs(dqk, dv, 300, 2.0 ** -4, 5000 + dqk, rising)
        for scale in (0.7, 10.0):
            for causal in (False, True):
                _check_all(q, k, v, causal, f"d{dqk} ramp rising={rising} scale={scale} causal={causal}",
                           scale=scale)


@pytest.mark.parametrize("dims", [(32, 32), (64, 64), (128, 128), (192, 128)])
def test_late_score_spike_overflows_the_reference(dims):
    # One key late in the sequence scores ~150 (natural-log units) above every other key, for every
    # query: against the reference max taken from the first block its probability overflows fp32
    # (2^216), so the block must take the rare path that moves the reference (for d128/d192 after
    # recomputing the block's scores from K in global memory) and redo its exponentials.  Keys
    # before the spike keep their tiny weights relative to it.  Key 3 is the same case for the
    # light block of a causal pair, which runs its tiles downward and meets key 3 in its last block.
    dqk, dv = dims
    s = 300
    q = workloads.make_random((1, s, 2, dqk), 8100 + dqk, dtype=torch.float32, std=0.1)
    k = workloads.make_random((1, s, 2, dqk), 8101 + dqk, dtype=torch.float32, std=0.1)
    q[..., 0] = 1.0
    for spike in (257, 100, 3):
        k2 = k.clone()
        k2[0, spike, :, 0] = 150.0 * dqk ** 0.5
        v = workloads.make_random((1, s, 2, dv), 8102 + dqk)
        for causal in (False, True):
            _check_all(q.to(torch.bfloat16), k2.to(torch.bfloat16), v, causal,
                       f"d{dqk} spike at key {spike} causal={causal}")
