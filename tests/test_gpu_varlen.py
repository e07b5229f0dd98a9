"""GPU parity of mha_fwd_bf16_varlen (packed sequences) against the float64 oracle (needs an MI355X)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_bf16_parity, require_gpu, to_np

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (128, 128), (192, 128)]


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _run(q, k, v, lens_q, lens_k, causal, scale, max_q=None, max_k=None):
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    cu_q = torch.from_numpy(_cu(lens_q)).to(dev)
    cu_k = torch.from_numpy(_cu(lens_k)).to(dev)
    mq = max(lens_q) if max_q is None else max_q
    mk = max(lens_k) if max_k is None else max_k
    o, lse = mha.mha_fwd_bf16_varlen(q.to(dev), k.to(dev), v.to(dev), cu_q, cu_k, mq, mk, causal=causal,
                                     softmax_scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _inputs(lens_q, lens_k, hq, hk, dqk, dv, seed):
    q = workloads.make_random((sum(lens_q), hq, dqk), seed)
    k = workloads.make_random((sum(lens_k), hk, dqk), seed + 1)
    v = workloads.make_random((sum(lens_k), hk, dv), seed + 2)
    return q, k, v


def _check(q, k, v, lens_q, lens_k, causal, what, **kw):
    dqk = q.shape[2]
    scale = dqk ** -0.5
    o, lse = _run(q, k, v, lens_q, lens_k, causal, scale, **kw)
    o_ref, l_ref = oracle.attention_varlen(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                           _cu(lens_q), _cu(lens_k), scale=scale, causal=causal)
    assert_bf16_parity(to_np(o), o_ref, lse.numpy().astype(np.float64), l_ref, what)
    return o, lse


@pytest.mark.parametrize("lens, causal", [([200, 333, 90], False), ([200, 333, 90], True), ([200, 150], True)],
                         ids=["3seq", "3seq-causal", "2seq-causal-paired"])
def test_two_heads_per_workgroup(lens, causal):
    # d128 GQA packed grids that still fill the device take two query heads per workgroup
    # (hq 512 over hk 256); the two-sequence causal grid is small enough to pair its blocks too.
    # V is drawn at half width: over these 23M outputs, causal rows that see one to three keys
    # and V values near 4 can move O by more than the flat 1e-2 through the bf16 rounding of P
    # (1.03e-2 with N(0, 1) values, the same bit for bit without the packing); the point here is
    # the packed path.
    q, k, _ = _inputs(lens, lens, 512, 256, 128, 128, 4500 + len(lens) + int(causal))
    v = workloads.make_random((sum(lens), 256, 128), 4502 + len(lens) + int(causal), std=0.5)
    _check(q, k, v, lens, lens, causal, f"varlen two heads per workgroup {lens} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dims", DIMS, ids=[f"d{a}-{b}" for a, b in DIMS])
def test_ragged_lengths(dims, causal):
    # lengths below, at and above the 128/256-row query blocks and the 64-key tiles
    dqk, dv = dims
    lens = [1, 127, 128, 300, 5, 257]
    q, k, v = _inputs(lens, lens, 4, 2, dqk, dv, 4000 + dqk + int(causal))
    _check(q, k, v, lens, lens, causal, f"varlen d{dqk} causal={causal}")


@pytest.mark.parametrize("dims", DIMS, ids=[f"d{a}-{b}" for a, b in DIMS])
def test_unequal_query_and_key_lengths(dims):
    # per sequence sq != sk, a sequence without keys (O = 0, LSE = -inf) and one without queries
    dqk, dv = dims
    lens_q = [40, 200, 0, 77, 129]
    lens_k = [300, 33, 64, 0, 129]
    q, k, v = _inputs(lens_q, lens_k, 6, 3, dqk, dv, 4100 + dqk)
    for causal in (False, True):
        o, lse = _check(q, k, v, lens_q, lens_k, causal, f"varlen sq!=sk d{dqk} causal={causal}")
        r0 = sum(lens_q[:3])                      # the sequence with no keys
        assert torch.all(o[r0:r0 + lens_q[3]] == 0)
        assert torch.all(torch.isneginf(lse[:, r0:r0 + lens_q[3]]))


@pytest.mark.parametrize("dims", [(128, 128, 333), (192, 128, 700)], ids=["d128", "d192"])
def test_loose_maximum_and_equal_lengths_match_dense(dims):
    # equal lengths: the packed call must reproduce the dense call bit for bit, also when
    # max_seqlen is larger than every sequence (the packed grid then pairs other blocks: at d192
    # the light blocks' downward order must follow the sequence, not the grid)
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    d, dv, s = dims
    b, hq, hk = 3, 4, 2
    q = workloads.make_random((b, s, hq, d), 4200)
    k = workloads.make_random((b, s, hk, d), 4201)
    v = workloads.make_random((b, s, hk, dv), 4202)
    for causal in (False, True):
        od, ld = mha.mha_fwd_bf16(q.to(dev), k.to(dev), v.to(dev), causal=causal, n_split=1)
        ov, lv = _run(q.reshape(b * s, hq, d), k.reshape(b * s, hk, d), v.reshape(b * s, hk, dv), [s] * b,
                      [s] * b, causal, d ** -0.5, max_q=1000, max_k=1000)
        torch.cuda.synchronize()
        assert torch.equal(ov.reshape(b, s, hq, dv), od.cpu())
        assert torch.equal(lv.reshape(hq, b, s).permute(1, 0, 2), ld.cpu())


def test_strided_packed_qkv_view():
    # q, k, v as head-sliced views of one packed [tokens, 3, h, d] buffer
    dev = require_gpu()
    lens = [65, 190, 3]
    t, h, d = sum(lens), 4, 64
    qkv = workloads.make_random((t, 3, h, d), 4300)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    import head_attention_forward_flash_amd as mha
    cu = torch.from_numpy(_cu(lens)).to(dev)
    qkv_d = qkv.to(dev)
    o, lse = mha.mha_fwd_bf16_varlen(qkv_d[:, 0], qkv_d[:, 1], qkv_d[:, 2], cu, cu, max(lens), max(lens), causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q.float().numpy(), k.float().numpy(), v.float().numpy(), _cu(lens),
                                           _cu(lens), scale=d ** -0.5, causal=True)
    assert_bf16_parity(to_np(o.cpu()), o_ref, lse.cpu().numpy().astype(np.float64), l_ref, "varlen strided qkv")


def test_many_short_sequences_sampled():
    # 64 sequences of 1..2000 tokens (GQA 8:1, d128, causal): sampled rows of two heads
    rng = np.random.default_rng(17)
    lens = [int(x) for x in rng.integers(1, 2000, size=64)]
    q, k, v = _inputs(lens, lens, 16, 2, 128, 128, 4400)
    o, lse = _run(q, k, v, lens, lens, True, 128 ** -0.5)
    rows = workloads.sample_indices(sum(lens), 256, 18, include=[0, sum(lens) - 1])
    heads = [0, 15]
    o_ref, l_ref = oracle.attention_varlen(q.float().numpy(), k.float().numpy(), v.float().numpy(), _cu(lens),
                                           _cu(lens), scale=128 ** -0.5, causal=True, heads=heads, rows=rows)
    assert_bf16_parity(to_np(o[rows][:, heads]), o_ref, lse[heads][:, rows].numpy().astype(np.float64), l_ref,
                       "varlen 64 sequences")
