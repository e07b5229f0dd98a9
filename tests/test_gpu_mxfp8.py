"""GPU parity of the MXFP8 quantised call: E4M3 codes and E8M0 exponents (bit-exact), V values
(bit-exact) and attention against the same-quantisation oracle (needs an MI355X)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import FP8_REL_L2, assert_fp8_parity, require_gpu

pytestmark = pytest.mark.gpu


def _call(q, k, v, mu, causal):
    """Run mha_fwd_mxfp8 on device copies; return (o, lse, quantised tensors read back)."""
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    b, sq, hq, d = q.shape
    _, sk, hk, _ = k.shape
    mu_d = None if mu is None else torch.from_numpy(np.ascontiguousarray(mu, dtype=np.float32)).to(dev)
    o, lse, ws = mha.mha_fwd_mxfp8(q.to(dev), k.to(dev), v.to(dev), k_mean=mu_d, causal=causal)
    torch.cuda.synchronize()
    off = mha.mha_mxfp8_workspace_layout(b, hq, hk, sq, sk, d)
    nq, nk = (sq + 127) // 128, (sk + 127) // 128
    wsc = ws.cpu().numpy()

    def rows(i, heads, n, width, s):
        raw = wsc[off[i]: off[i] + b * heads * n * 128 * width].reshape(b, heads, n * 128, width)
        return raw[:, :, :s, :].transpose(0, 2, 1, 3), raw[:, :, s:, :]      # [b, s, h, w], padding

    qc, qpad = rows(0, hq, nq, d, sq)
    kc, kpad = rows(1, hk, nk, d, sk)
    qe, qepad = rows(3, hq, nq, d // 32, sq)
    ke, kepad = rows(4, hk, nk, d // 32, sk)
    vraw = ws[off[2]: off[2] + b * hk * nk * 128 * d * 2].view(torch.bfloat16).float().cpu().numpy()
    vvals = vraw.reshape(b, hk, nk * 128, d)[:, :, :sk, :].transpose(0, 2, 1, 3)
    quant = {"q": (qc, qe), "k": (kc, ke), "v": vvals}
    pads = (qpad, kpad, qepad, kepad)
    return o.cpu(), lse.cpu(), quant, pads


def _inputs(b, sq, sk, hq, hk, d, seed, bias_std=3.0):
    q = workloads.make_random((b, sq, hq, d), seed)
    k = workloads.make_random((b, sk, hk, d), seed + 1, dtype=torch.float32)
    bias = workloads.make_random((1, 1, hk, d), seed + 2, dtype=torch.float32) * bias_std
    k = (k + bias).to(torch.bfloat16)
    v = workloads.make_random((b, sk, hk, d), seed + 3)
    return q, k, v


def _oracle_mu(k):
    return oracle.k_smooth_mean(k.float().numpy())["mean"].astype(np.float32)


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("smooth", [True, False])
def test_codes_exponents_and_values_bit_exact(smooth, d):
    q, k, v = _inputs(2, 300, 200, 4, 2, d, 5000 + d)
    mu = _oracle_mu(k) if smooth else None
    _, _, quant, pads = _call(q, k, v, mu, causal=False)
    qc, qe, _ = oracle.mx_quantize(q.float().numpy())
    kc, ke, _ = oracle.mx_quantize(oracle.fp8.smooth_k(k.float().numpy(), mu))
    _, _, vv = oracle.mx_quantize(v.float().numpy())
    for name, (c_ref, e_ref) in (("q", (qc, qe)), ("k", (kc, ke))):
        c_gpu, e_gpu = quant[name]
        assert int((e_gpu != e_ref).sum()) == 0, f"{name}: exponent bytes differ"
        mism = int((c_gpu != c_ref).sum())
        assert mism == 0, f"{name}: {mism} of {c_ref.size} codes differ"
    np.testing.assert_array_equal(quant["v"].astype(np.float64), vv, err_msg="V values")
    assert all((pad == 0).all() for pad in pads), "token padding must be zero codes and exponent bytes"


def _check(q, k, v, mu, causal, what, heads=None, rows=None):
    o, lse, _, _ = _call(q, k, v, mu, causal)
    d = q.shape[3]
    o_ref, lse_ref, _ = oracle.mxfp8_attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                       mu=mu, scale=d ** -0.5, causal=causal, heads=heads, rows=rows)
    o_g = o.float().numpy().astype(np.float64)
    l_g = lse.numpy().astype(np.float64)
    if heads is not None:
        o_g, l_g = o_g[:, :, heads], l_g[:, heads]
    if rows is not None:
        o_g, l_g = o_g[:, rows], l_g[:, :, rows]
    assert_fp8_parity(o_g, o_ref, l_g, lse_ref, what)


def test_two_blocks_per_workgroup():
    # the packed non-causal d128 kernel (256 heads, odd block count) with E8M0 exponents
    q, k, v = _inputs(1, 300, 333, 256, 256, 128, 5300)
    _check(q, k, v, _oracle_mu(k), False, "mxfp8 two blocks per workgroup", heads=[0, 1, 128, 255])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_gqa(causal, d):
    q, k, v = _inputs(2, 300, 200, 4, 2, d, 5100 + d)
    _check(q, k, v, _oracle_mu(k), causal, f"ragged gqa d{d} causal={causal}")


def test_no_smoothing_and_negative_scale():
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    q, k, v = _inputs(1, 256, 384, 2, 2, 128, 5200, bias_std=0.0)
    _check(q, k, v, None, False, "no smoothing")
    # a negative softmax scale flips the sign of every score
    o, _, _ = mha.mha_fwd_mxfp8(q.to(dev), k.to(dev), v.to(dev), softmax_scale=-128 ** -0.5)
    torch.cuda.synchronize()
    o_ref, _, _ = oracle.mxfp8_attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                 scale=-128 ** -0.5, causal=False)
    assert _rel_l2(o.cpu().float().numpy(), o_ref) <= FP8_REL_L2


def test_large_and_small_magnitudes():
    # blocks whose exponents sit far from 0: K ~ 1e4, V ~ 1e-3
    q = workloads.make_random((1, 200, 2, 128), 5300, std=0.05)
    k = workloads.make_random((1, 200, 2, 128), 5301, std=3e3)
    v = workloads.make_random((1, 200, 2, 128), 5302, std=1e-3)
    _check(q, k, v, None, True, "large/small magnitudes")


def test_full_workload_sampled_heads():
    w = workloads.WORKLOADS["mxfp8_ksmooth_d128"]
    q, k, v = workloads.make_qkv(w)
    _check(q, k, v, _oracle_mu(k), w.causal, "mxfp8 workload", heads=[0, 9, 15])


def test_gpu_gate_then_mxfp8_matches_oracle_pipeline():
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    q, k, v = _inputs(1, 512, 512, 4, 4, 128, 5400)
    kd = k.to(dev)
    mean, gate = mha.k_smooth_mean(kd)
    o, lse, _ = mha.mha_fwd_mxfp8(q.to(dev), kd, v.to(dev), k_mean=mean)
    torch.cuda.synchronize()
    assert gate.cpu().numpy().all()
    o_ref, lse_ref, _ = oracle.mxfp8_attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                       mu=_oracle_mu(k), scale=128 ** -0.5, causal=False)
    assert_fp8_parity(o.cpu().float().numpy().astype(np.float64), o_ref, lse.cpu().numpy().astype(np.float64),
                      lse_ref, "gate+mxfp8 pipeline")


def test_mxfp8_deterministic():
    q, k, v = _inputs(1, 400, 400, 2, 2, 128, 5500)
    mu = _oracle_mu(k)
    a = _call(q, k, v, mu, True)
    b = _call(q, k, v, mu, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_late_score_spike_overflows_the_reference():
    d, s = 128, 384
    q = workloads.make_random((1, s, 2, d), 8300, dtype=torch.float32, std=0.1)
    k = workloads.make_random((1, s, 2, d), 8301, dtype=torch.float32, std=0.1)
    q[..., 0] = 1.0
    k[0, 300, :, 0] = 150.0 * d ** 0.5
    v = workloads.make_random((1, s, 2, d), 8302)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    for causal in (False, True):
        _check(q, k, v, None, causal, f"spike causal={causal}")
