"""GPU parity of k_smooth_mean against the float64 gate oracle (needs an MI355X)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import require_gpu

pytestmark = pytest.mark.gpu


def _gate(k, **kw):
    import head_attention_forward_flash_amd as mha
    mean, gate = mha.k_smooth_mean(k, **kw)
    torch.cuda.synchronize()
    return mean.cpu().numpy().astype(np.float64), gate.cpu().numpy()


def _check(k_dev, what, key_stride=1, max_keys=0, tau=0.25):
    mean, gate = _gate(k_dev, key_stride=key_stride, max_keys=max_keys, tau=tau)
    ref = oracle.k_smooth_mean(k_dev.float().cpu().numpy(), key_stride=key_stride, max_keys=max_keys, tau=tau)
    np.testing.assert_array_equal(gate.astype(bool), ref["open"], err_msg=what)
    tol = 1e-5 * (1.0 + np.abs(ref["mu"]).max())
    err = np.abs(mean - ref["mean"]).max() if mean.size else 0.0
    print(f"[gate] {what}: max|mu err|={err:.3e} open={int(gate.sum())}/{gate.size}", flush=True)
    assert err <= tol, f"{what}: mean error {err} > {tol}"
    assert (mean[~ref["open"]] == 0.0).all()
    return mean, gate, ref


def test_fp8_workload_gate_open_everywhere():
    dev = require_gpu()
    w = workloads.WORKLOADS["fp8_ksmooth_d128"]
    _, k, _ = workloads.make_qkv(w)
    _, gate, ref = _check(k.to(dev), "fp8 workload K (bias std 3)")
    assert gate.all()


def test_unbiased_k_gate_closed_everywhere():
    dev = require_gpu()
    w = workloads.WORKLOADS["fp8_ksmooth_d128"]
    _, k, _ = workloads.make_qkv(w, k_bias_std=0.0)
    _, gate, _ = _check(k.to(dev), "fp8 workload K without bias")
    assert not gate.any()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("stride,max_keys", [(1, 0), (3, 0), (5, 100), (1, 700), (4096, 0)])
def test_strided_and_partial_samples(d, stride, max_keys):
    dev = require_gpu()
    b, sk, hk = 2, 1500, 3
    k = workloads.make_random((b, sk, hk, d), 100 + d + stride)
    bias = workloads.make_random((1, 1, hk, d), 200 + d, dtype=torch.float32)
    bias[:, :, 1] = 0.0                  # kv head 1 stays unbiased: its gate closes
    k = (k.float() + 2.0 * bias).to(torch.bfloat16)
    _check(k.to(dev), f"d={d} stride={stride} max_keys={max_keys}", key_stride=stride, max_keys=max_keys)


def test_head_sliced_and_misaligned_views():
    dev = require_gpu()
    base = workloads.make_random((1, 777, 5, 130), 300, std=1.0, mean=0.5).to(dev)
    sliced = base[:, :, 1:4, 0:128]            # head-sliced view, aligned rows (stride 650)
    mis = base[:, :, 1:4, 1:129]               # starts 2 bytes in: scalar-load path
    m_ref, g_ref = _gate(sliced.contiguous())
    for view, what in ((sliced, "head-sliced"), (mis, "misaligned")):
        _check(view, what)
    m1, g1 = _gate(sliced)
    np.testing.assert_array_equal(m1, m_ref)
    np.testing.assert_array_equal(g1, g_ref)


def test_gate_outcomes_and_determinism():
    dev = require_gpu()
    k = workloads.make_random((3, 1000, 2, 128), 400).to(dev)
    k[0] += 5.0                                   # batch 0: large mean, open
    k[1, 1::2] = -k[1, 0::2]                      # batch 1: paired keys, mean 0, closed
    mean, gate, ref = _check(k, "outcomes")
    assert gate[0].all() and not gate[1].any()
    m2, g2 = _gate(k)
    np.testing.assert_array_equal(mean, m2)
    np.testing.assert_array_equal(gate, g2)


def test_empty_keys():
    dev = require_gpu()
    k = torch.empty((2, 0, 2, 64), dtype=torch.bfloat16, device=dev)
    mean, gate = _gate(k)
    assert (mean == 0).all() and (gate == 0).all()
