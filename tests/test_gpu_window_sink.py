"""GPU parity of sliding-window / sink attention and of the d32 head size against the float64
oracles (needs an MI355X)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_bf16_parity, require_gpu, to_np

pytestmark = pytest.mark.gpu

DIMS = [(32, 32), (64, 64), (128, 128), (192, 128)]


def _inputs(b, sq, sk, hq, hk, dqk, dv, seed):
    q = workloads.make_random((b, sq, hq, dqk), seed)
    k = workloads.make_random((b, sk, hk, dqk), seed + 1)
    v = workloads.make_random((b, sk, hk, dv), seed + 2)
    return q, k, v


def _run(q, k, v, causal, left, right, sinks, scale=None):
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    s_d = None if sinks is None else torch.as_tensor(sinks, dtype=torch.float32).to(dev)
    o, lse = mha.mha_fwd_bf16_window_sink(q.to(dev), k.to(dev), v.to(dev), causal=causal, window_left=left,
                                          window_right=right, sinks=s_d, softmax_scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check(q, k, v, causal, left, right, sinks, what, rows=None, heads=None, scale=None):
    scale = q.shape[3] ** -0.5 if scale is None else scale
    o, lse = _run(q, k, v, causal, left, right, sinks, scale)
    o_ref, l_ref = oracle.attention_window_sink(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                scale=scale, causal=causal, window_left=left, window_right=right,
                                                sinks=None if sinks is None else np.asarray(sinks, np.float64),
                                                rows=rows, heads=heads)
    o_g, l_g = to_np(o), lse.numpy().astype(np.float64)
    if heads is not None:
        o_g, l_g = o_g[:, :, heads], l_g[:, heads]
    if rows is not None:
        o_g, l_g = o_g[:, rows], l_g[:, :, rows]
    assert_bf16_parity(o_g, o_ref, l_g, l_ref, what)


@pytest.mark.parametrize("dims", DIMS, ids=[f"d{a}-{b}" for a, b in DIMS])
@pytest.mark.parametrize("causal,left,right", [(True, 100, -1), (True, 0, -1), (False, 70, 33), (False, -1, 0),
                                               (True, 300, -1)])
def test_window_ragged_gqa(dims, causal, left, right):
    dqk, dv = dims
    q, k, v = _inputs(2, 333, 333, 4, 2, dqk, dv, 6000 + dqk + left)
    _check(q, k, v, causal, left, right, None, f"window d{dqk} causal={causal} ({left},{right})")


@pytest.mark.parametrize("dims", DIMS, ids=[f"d{a}-{b}" for a, b in DIMS])
def test_sinks_with_and_without_window(dims):
    dqk, dv = dims
    q, k, v = _inputs(1, 290, 290, 6, 3, dqk, dv, 6100 + dqk)
    sinks = np.array([-1.0, 0.0, 0.5, 2.0, 8.0, -30.0], dtype=np.float32)
    for causal, left in ((True, -1), (False, -1), (True, 127)):
        _check(q, k, v, causal, left, -1, sinks, f"sinks d{dqk} causal={causal} left={left}")


def test_sink_dominates_and_rows_without_keys():
    # huge sinks drive O to 0 and LSE to the sink; sq > sk with a right window leaves late rows
    # without keys: O = 0, LSE = sink
    q, k, v = _inputs(1, 260, 70, 2, 1, 64, 64, 6200)
    sinks = np.array([40.0, 0.25], dtype=np.float32)
    _check(q, k, v, False, 10, 0, sinks, "rows without keys, big sink")
    o, lse = _run(q, k, v, False, 10, 0, sinks)
    assert torch.all(o[0, 80:] == 0)
    assert torch.all((lse[0, 1, 80:] - 0.25).abs() <= 1e-6)


def test_minus_inf_sinks_and_wide_window_match_the_plain_kernel():
    # the windowed kernel with sinks of -inf and a window wider than the sequence reproduces the
    # plain kernel's O bit for bit; its LSE may round the max's product once more (one ulp)
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    q, k, v = _inputs(2, 300, 300, 4, 2, 128, 128, 6300)
    for causal in (False, True):
        op, lp = mha.mha_fwd_bf16(q.to(dev), k.to(dev), v.to(dev), causal=causal)
        ow, lw = _run(q, k, v, causal, 299, -1 if causal else 299, np.full(4, -np.inf, np.float32))
        torch.cuda.synchronize()
        assert torch.equal(op.cpu(), ow)
        torch.testing.assert_close(lw, lp.cpu(), rtol=2.0 ** -22, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_d32_dense_and_varlen(causal):
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    q, k, v = _inputs(2, 300, 300, 4, 2, 32, 32, 6400 + int(causal))
    o, lse = mha.mha_fwd_bf16(q.to(dev), k.to(dev), v.to(dev), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                            scale=32 ** -0.5, causal=causal)
    assert_bf16_parity(to_np(o.cpu()), o_ref, lse.cpu().numpy().astype(np.float64), l_ref, f"d32 causal={causal}")
    lens = [1, 200, 129, 64]
    qv, kv, vv = (workloads.make_random((sum(lens), h, 32), 6500 + i) for i, h in enumerate((4, 2, 2)))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    ov, lv = mha.mha_fwd_bf16_varlen(qv.to(dev), kv.to(dev), vv.to(dev), cu, cu, max(lens), max(lens), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(qv.float().numpy(), kv.float().numpy(), vv.float().numpy(), cu.cpu().numpy(),
                                           cu.cpu().numpy(), scale=32 ** -0.5, causal=causal)
    assert_bf16_parity(to_np(ov.cpu()), o_ref, lv.cpu().numpy().astype(np.float64), l_ref, f"d32 varlen causal={causal}")


def test_gptoss_window_workload_sampled():
    w = workloads.WORKLOADS["gptoss_swa_sink_d64"]
    q, k, v = workloads.make_qkv(w)
    sinks = workloads.make_sinks(w).numpy()
    rows = workloads.sample_indices(w.sq, 160, 21, include=[0, 126, 127, 128, 4095, w.sq - 1])
    _check(q, k, v, w.causal, w.window_left, w.window_right, sinks, "gpt-oss window layer", rows=rows,
           heads=[0, 13, 63])


def test_gptoss_full_sink_workload_sampled():
    w = workloads.WORKLOADS["gptoss_sink_d64"]
    q, k, v = workloads.make_qkv(w)
    sinks = workloads.make_sinks(w).numpy()
    rows = workloads.sample_indices(w.sq, 96, 22, include=[0, 1, w.sq - 1])
    _check(q, k, v, w.causal, -1, -1, sinks, "gpt-oss full layer", rows=rows, heads=[5, 40])


@pytest.mark.parametrize("dims", [(64, 64), (128, 128)], ids=["d64", "d128"])
@pytest.mark.parametrize("causal,left,right", [(True, 127, -1), (False, 40, 25)])
def test_packed_sequences_with_window_and_sinks(dims, causal, left, right):
    # positions restart per sequence; lengths below, at and above the 128-row blocks
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    dqk, dv = dims
    lens = [1, 300, 129, 77, 128]
    q = workloads.make_random((sum(lens), 4, dqk), 6600 + dqk)
    k = workloads.make_random((sum(lens), 2, dqk), 6601 + dqk)
    v = workloads.make_random((sum(lens), 2, dv), 6602 + dqk)
    sinks = np.array([0.3, -2.0, 1.5, 0.0], dtype=np.float32)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    o, lse = mha.mha_fwd_bf16_varlen(q.to(dev), k.to(dev), v.to(dev), cu, cu, max(lens), max(lens), causal=causal,
                                     window_left=left, window_right=right, sinks=torch.from_numpy(sinks).to(dev))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen_window_sink(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                       cu.cpu().numpy(), cu.cpu().numpy(), scale=dqk ** -0.5,
                                                       causal=causal, window_left=left, window_right=right,
                                                       sinks=sinks.astype(np.float64))
    assert_bf16_parity(to_np(o.cpu()), o_ref, lse.cpu().numpy().astype(np.float64), l_ref,
                       f"packed window d{dqk} causal={causal} ({left},{right})")


@pytest.mark.parametrize("dims", [(64, 64), (128, 128)], ids=["d64", "d128"])
@pytest.mark.parametrize("causal,left,right", [(True, -1, -1), (False, -1, 33), (False, -1, -1), (True, 100, -1)])
def test_two_heads_per_workgroup_window_sinks(dims, causal, left, right):
    # GQA grids that fill the device (hq 512 over hk 256, 3 blocks of 128 rows) run two query
    # heads per workgroup with sinks and right windows too: each wave takes its own head's sink
    # and its own rows' window; both heads of a workgroup (even and odd) are checked, dense and
    # packed.  (A left window keeps one head per workgroup: the last case.)
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    dqk, dv = dims
    heads = [0, 1, 2, 3, 100, 257, 510, 511]
    sinks = workloads.make_random((512,), 6700 + dqk, dtype=torch.float32, std=2.0).numpy()
    q, k, v = _inputs(1, 300, 300, 512, 256, dqk, dv, 6710 + dqk + left)
    _check(q, k, v, causal, left, right, sinks, f"two heads window d{dqk} causal={causal} ({left},{right})",
           heads=heads)
    lens = [200, 333, 90]
    q = workloads.make_random((sum(lens), 512, dqk), 6720 + dqk)
    k = workloads.make_random((sum(lens), 256, dqk), 6721 + dqk)
    v = workloads.make_random((sum(lens), 256, dv), 6722 + dqk)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    o, lse = mha.mha_fwd_bf16_varlen(q.to(dev), k.to(dev), v.to(dev), cu, cu, max(lens), max(lens), causal=causal,
                                     window_left=left, window_right=right, sinks=torch.from_numpy(sinks).to(dev))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen_window_sink(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                       cu.cpu().numpy(), cu.cpu().numpy(), scale=dqk ** -0.5,
                                                       causal=causal, window_left=left, window_right=right,
                                                       sinks=sinks.astype(np.float64), heads=heads)
    assert_bf16_parity(to_np(o.cpu())[:, heads], o_ref, lse.cpu().numpy().astype(np.float64)[heads], l_ref,
                       f"two heads packed window d{dqk} causal={causal} ({left},{right})")


@pytest.mark.parametrize("hq,hk", [(4, 2), (512, 256)], ids=["one-head", "two-heads"])
def test_negative_scale_with_window_and_sinks(hq, hk):
    # a negative scale flips Q's sign in every block's prologue, in the window/sink kernels too
    # (hq 512 over hk 256 with sinks and no left window takes the two-heads-per-workgroup kernel)
    heads = None if hq == 4 else [0, 1, 255, 510, 511]
    sinks = workloads.make_random((hq,), 6800 + hq, dtype=torch.float32, std=2.0).numpy()
    q, k, v = _inputs(1, 300, 300, hq, hk, 64, 64, 6810 + hq)
    _check(q, k, v, True, -1, -1, sinks, f"scale=-0.2 sinks hq={hq}", heads=heads, scale=-0.2)
    _check(q, k, v, True, 100, -1, sinks, f"scale=-0.2 window sinks hq={hq}", heads=heads, scale=-0.2)
