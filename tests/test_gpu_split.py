"""GPU parity of the key-range split (mha_fwd_bf16_split) against the float64 oracle.

Each query block's keys are divided among n_split workgroups whose partial states a second
kernel merges; the oracle knows nothing of the split, so these tests check that the ranges
cover every key once, that the merge weights are right (including ranges whose maxima lie far
apart) and that nothing depends on what the workspace held before the call.
"""

import numpy as np
import pytest
import torch

import workloads
from parity import assert_bf16_parity, oracle_heads, require_gpu, scale_for, to_np

pytestmark = pytest.mark.gpu

SPLIT_SHAPES = [
    # b, hq, hk, sq, sk, d_qk, d_v, n_split
    (1, 2, 1, 200, 1000, 32, 32, 3),       # 16 key tiles -> 5/5/6, ragged tail (1000 = 15*64 + 40)
    (2, 3, 1, 130, 777, 64, 64, 5),        # 13 tiles -> 2/3/2/3/3, two query blocks (ragged)
    (1, 4, 2, 257, 1100, 128, 128, 2),     # GQA 2:1, three query blocks
    (1, 5, 1, 128, 640, 128, 128, 10),     # GQA 5:1, one tile per range
    (1, 2, 2, 300, 700, 192, 128, 4),      # 256-row blocks of 8 waves
    (1, 2, 1, 64, 4096, 128, 128, 16),     # the largest split, 4 tiles per range
]


def _lib():
    import head_attention_forward_flash_amd as mha
    return mha


def _inputs(shape, seed):
    b, hq, hk, sq, sk, dqk, dv, _ = shape
    q = workloads.make_random((b, sq, hq, dqk), seed)
    k = workloads.make_random((b, sk, hk, dqk), seed + 1)
    v = workloads.make_random((b, sk, hk, dv), seed + 2)
    return q, k, v


def _run(q, k, v, n_split, workspace=None, scale=None):
    dev = require_gpu()
    o, lse = _lib().mha_fwd_bf16(q.to(dev), k.to(dev), v.to(dev), causal=False, softmax_scale=scale,
                                 n_split=n_split, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check(q, k, v, o, lse, scale, what):
    b, hq = q.shape[0], q.shape[2]
    for bb in range(b):
        o_ref, l_ref = oracle_heads(q, k, v, list(range(hq)), None, scale=scale, causal=False, batch=bb)
        assert_bf16_parity(to_np(o[bb]), o_ref, lse[bb].numpy().astype(np.float64), l_ref, f"{what} b={bb}")


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=[f"b{s[0]}h{s[1]}/{s[2]}q{s[3]}k{s[4]}d{s[5]}-{s[6]}x{s[7]}"
                                                      for s in SPLIT_SHAPES])
def test_split_matches_oracle(shape):
    q, k, v = _inputs(shape, 2000 + sum(shape))
    o, lse = _run(q, k, v, shape[-1])
    _check(q, k, v, o, lse, scale_for(shape[5]), f"split {shape}")


def test_split_is_deterministic_and_ignores_workspace_contents():
    # every workspace word the merge reads is written by the same call, whatever the workspace
    # held; the merge adds the ranges in one fixed order
    dev = require_gpu()
    shape = (1, 5, 1, 640, 2048, 128, 128, 6)
    q, k, v = _inputs(shape, 77)
    b, hq, hk, sq, sk, dqk, dv, n = shape
    need = _lib().mha_fwd_bf16_split_workspace_bytes(b, hq, sq, dqk, dv, n)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    first = _run(q, k, v, n, workspace=ws)
    for fill in (0x00, 0x7F):
        ws.fill_(fill)
        again = _run(q, k, v, n, workspace=ws)
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1]), fill
    _check(q, k, v, first[0], first[1], scale_for(dqk), "deterministic split")


def test_split_workspace_reused_by_a_smaller_call():
    # one workspace, two calls in a row on the stream: the second (fewer blocks, another split)
    # finds the first call's partials and must not be confused by them
    dev = require_gpu()
    big = (2, 4, 2, 384, 1500, 64, 64, 7)
    small = (1, 2, 2, 130, 900, 64, 64, 3)
    need = _lib().mha_fwd_bf16_split_workspace_bytes(2, 4, 384, 64, 64, 7)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    for shape, seed in ((big, 91), (small, 92)):
        q, k, v = _inputs(shape, seed)
        o, lse = _run(q, k, v, shape[-1], workspace=ws)
        _check(q, k, v, o, lse, scale_for(shape[5]), f"reused workspace {shape}")


@pytest.mark.parametrize("dims", [(32, 32), (64, 64), (128, 128), (192, 128)])
def test_split_ranges_far_apart(dims):
    # Query channel 0 is 1 and one key scores ~150 above the rest, in the middle range of three:
    # the other ranges' weights 2^(m_i - M) underflow to 0 in the merge.  A key ~150 below the
    # rest sits in the first range, whose max stays that of the ordinary keys.
    dqk, dv = dims
    sq, sk, n = 160, 960, 3
    q = workloads.make_random((1, sq, 2, dqk), 61 + dqk).float()
    k = workloads.make_random((1, sk, 1, dqk), 62 + dqk).float()
    v = workloads.make_random((1, sk, 1, dv), 63 + dqk)
    q[..., 0] = 1.0
    k[0, 480, :, 0] = 150.0 * dqk ** 0.5
    k[0, 100, :, 0] = -150.0 * dqk ** 0.5
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o, lse = _run(q, k, v, n)
    _check(q, k, v, o, lse, scale_for(dqk), f"spiked split d{dqk}")


def test_split_against_unsplit_and_plan():
    dev = require_gpu()
    mha = _lib()
    # the TP8 rank shapes: 320 query blocks of GQA 5:1 leave most compute units with one
    # workgroup, so the plan splits them; 512 blocks of GQA 8:1 fill the device, so it does not
    n5 = mha.mha_fwd_bf16_split_plan(1, 5, 1, 8192, 8192, 128, 128, False)
    n8 = mha.mha_fwd_bf16_split_plan(1, 8, 1, 8192, 8192, 128, 128, False)
    assert n5 > 1 and n8 == 1, (n5, n8)
    assert mha.mha_fwd_bf16_split_plan(1, 2, 2, 128, 128, 64, 64, False) == 1   # two key tiles
    # The same inputs through both kernels.  They differ in which reference max each probability
    # is rounded to bf16 against (the row sum adds the rounded values), so ln l moves by the
    # random bf16 rounding of thousands of terms: the oracle's LSE bound, 2^-8, holds for both.
    shape = (1, 5, 1, 512, 3000, 128, 128, n5)
    q, k, v = _inputs(shape, 88)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = mha.mha_fwd_bf16(qd, kd, vd, n_split=1)
    o2, l2 = mha.mha_fwd_bf16(qd, kd, vd, n_split=n5)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2.0 ** -7
    assert (l1 - l2).abs().max().item() <= 2.0 ** -8


def test_split_on_strided_views():
    # q, k, v as head slices of wider tensors and o written into a slice of a wider buffer: the
    # split kernel takes the same strides as the unsplit one
    dev = require_gpu()
    mha = _lib()
    base_q = workloads.make_random((2, 300, 6, 64), 71)
    base_k = workloads.make_random((2, 900, 4, 64), 72)
    base_v = workloads.make_random((2, 900, 4, 64), 73)
    q, k, v = base_q[:, :, 1:4], base_k[:, :, 2:3], base_v[:, :, 0:1]
    out_buf = torch.zeros((2, 300, 8, 64), dtype=torch.bfloat16, device=dev)
    out = out_buf[:, :, 2:5]
    o, lse = mha.mha_fwd_bf16(base_q.to(dev)[:, :, 1:4], base_k.to(dev)[:, :, 2:3], base_v.to(dev)[:, :, 0:1],
                              out=out, n_split=4)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    ob = out_buf.cpu()
    assert torch.all(ob[:, :, :2] == 0) and torch.all(ob[:, :, 5:] == 0)
    _check(q, k, v, ob[:, :, 2:5], lse.cpu(), scale_for(64), "strided split")


CAUSAL_SPLIT_SHAPES = [
    # b, hq, hk, sq, sk, d_qk, d_v, n_split
    (1, 2, 1, 1000, 1000, 128, 128, 2),    # 8 blocks, 4 pairs of 18 tiles: ranges of 9 cross blocks
    (1, 2, 1, 1000, 1000, 128, 128, 5),    # ranges of 3-4 tiles, some starting in diagonal tiles
    (1, 2, 1, 1000, 1000, 128, 128, 16),   # the largest n_split the call takes: ranges of 1-2 tiles
    (2, 3, 1, 520, 520, 64, 64, 3),        # 5 blocks: pairs (4, 0), (3, 1) and the middle block alone
    (1, 2, 2, 900, 900, 192, 128, 4),      # 256-row blocks: pairs (3, 0), (2, 1)
    (1, 4, 2, 300, 300, 32, 32, 4),        # d32: 3 blocks, the shortest pair 4 tiles
    (1, 2, 1, 600, 900, 128, 128, 3),      # more keys than queries: keys past a block's rows unseen
    (1, 2, 1, 900, 600, 128, 128, 3),      # fewer keys: the late blocks' tiles saturate at 10
]


@pytest.mark.parametrize("shape", CAUSAL_SPLIT_SHAPES,
                         ids=[f"b{s[0]}h{s[1]}/{s[2]}q{s[3]}k{s[4]}d{s[5]}-{s[6]}x{s[7]}" for s in CAUSAL_SPLIT_SHAPES])
def test_causal_split_matches_oracle(shape):
    dev = require_gpu()
    q, k, v = _inputs(shape, 3000 + sum(shape))
    o, lse = _lib().mha_fwd_bf16(q.to(dev), k.to(dev), v.to(dev), causal=True, n_split=shape[-1])
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    b, hq = q.shape[0], q.shape[2]
    scale = scale_for(shape[5])
    for bb in range(b):
        o_ref, l_ref = oracle_heads(q, k, v, list(range(hq)), None, scale=scale, causal=True, batch=bb)
        assert_bf16_parity(to_np(o[bb]), o_ref, lse[bb].numpy().astype(np.float64), l_ref,
                           f"causal split {shape} b={bb}")


def test_causal_split_deterministic_and_spiked():
    # a key ~150 above the rest inside the second block of a pair's sequence, and a rerun on a
    # workspace filled with other bytes: the same bits
    dev = require_gpu()
    q = workloads.make_random((1, 1000, 2, 128), 81).float()
    k = workloads.make_random((1, 1000, 1, 128), 82).float()
    v = workloads.make_random((1, 1000, 1, 128), 83)
    q[..., 0] = 1.0
    k[0, 40, :, 0] = 150.0 * 128 ** 0.5     # in block 0, the second block of pair (7, 0)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    mha = _lib()
    need = mha.mha_fwd_bf16_split_workspace_bytes(1, 2, 1000, 128, 128, 5)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev)
    first = mha.mha_fwd_bf16(q.to(dev), k.to(dev), v.to(dev), causal=True, n_split=5, workspace=ws)
    ws.fill_(0xA5)
    again = mha.mha_fwd_bf16(q.to(dev), k.to(dev), v.to(dev), causal=True, n_split=5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])
    o_ref, l_ref = oracle_heads(q, k, v, [0, 1], None, scale=scale_for(128), causal=True, batch=0)
    assert_bf16_parity(to_np(first[0].cpu()[0]), o_ref, first[1].cpu()[0].numpy().astype(np.float64), l_ref,
                       "causal split with a spike")


def test_causal_split_plan():
    mha = _lib()
    # causal 8192^2 d128 per-rank shapes: hq8/hk1 makes 256 pairs, one per CU, where a lone
    # workgroup already gets most of the CU (measured: every split slower) -> no split; hq5/hk1
    # leaves 96 CUs idle and hq1 most of the device -> split
    assert mha.mha_fwd_bf16_split_plan(1, 8, 1, 8192, 8192, 128, 128, True) == 1
    assert mha.mha_fwd_bf16_split_plan(1, 5, 1, 8192, 8192, 128, 128, True) > 1
    assert mha.mha_fwd_bf16_split_plan(1, 1, 1, 8192, 8192, 128, 128, True) > 1
    # the d128 GQA 4096^2 causal shape: 512 pairs fill the device -> no split
    assert mha.mha_fwd_bf16_split_plan(1, 32, 8, 4096, 4096, 128, 128, True) == 1
    # the MLA shape and its TP8 share: 256-row blocks of 8 waves -> no split
    assert mha.mha_fwd_bf16_split_plan(1, 128, 128, 8192, 8192, 192, 128, True) == 1
    assert mha.mha_fwd_bf16_split_plan(1, 16, 16, 8192, 8192, 192, 128, True) == 1
