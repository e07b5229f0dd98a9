"""GPU parity of the quantised path: E4M3 block codes (bit-exact) and FP8 attention (needs an MI355X)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import assert_fp8_parity, require_gpu

pytestmark = pytest.mark.gpu


def _fp8_call(q, k, v, mu, causal):
    """Run mha_fwd_fp8 on device copies; return (o, lse, quantised tensors read back from the workspace)."""
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    b, sq, hq, d = q.shape
    _, sk, hk, _ = k.shape
    mu_d = None if mu is None else torch.from_numpy(np.ascontiguousarray(mu, dtype=np.float32)).to(dev)
    o, lse, ws = mha.mha_fwd_fp8(q.to(dev), k.to(dev), v.to(dev), k_mean=mu_d, causal=causal)
    torch.cuda.synchronize()
    off = mha.mha_fp8_workspace_layout(b, hq, hk, sq, sk, d)
    nq, nk = (sq + 127) // 128, (sk + 127) // 128
    wsc = ws.cpu().numpy()

    def codes(i, heads, n, s):
        raw = wsc[off[i]: off[i] + b * heads * n * 128 * d].reshape(b, heads, n * 128, d)
        return raw[:, :, :s, :].transpose(0, 2, 1, 3)          # -> [b, s, h, d]

    def widened(i, heads, n, s):
        # V is stored as its E4M3 values widened to bf16: return the codes those values encode
        raw = ws[off[i]: off[i] + b * heads * n * 128 * d * 2].view(torch.bfloat16).float().cpu().numpy()
        vals = raw.reshape(b, heads, n * 128, d)[:, :, :s, :].transpose(0, 2, 1, 3)
        return oracle.e4m3_encode(vals.astype(np.float64))

    def scales(i, heads, n):
        return wsc[off[i]: off[i] + b * heads * n * 4].view(np.float32).reshape(b, heads, n)

    quant = {"q": (codes(0, hq, nq, sq), scales(3, hq, nq)), "k": (codes(1, hk, nk, sk), scales(4, hk, nk)),
             "v": (widened(2, hk, nk, sk), scales(5, hk, nk))}
    pad = {"q": wsc[off[0]: off[0] + b * hq * nq * 128 * d].reshape(b, hq, nq * 128, d)[:, :, sq:],
           "k": wsc[off[1]: off[1] + b * hk * nk * 128 * d].reshape(b, hk, nk * 128, d)[:, :, sk:]}
    return o.cpu(), lse.cpu(), quant, pad


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _inputs(b, sq, sk, hq, hk, d, seed, bias_std=3.0):
    q = workloads.make_random((b, sq, hq, d), seed)
    k = workloads.make_random((b, sk, hk, d), seed + 1, dtype=torch.float32)
    bias = workloads.make_random((1, 1, hk, d), seed + 2, dtype=torch.float32) * bias_std
    k = (k + bias).to(torch.bfloat16)
    v = workloads.make_random((b, sk, hk, d), seed + 3)
    return q, k, v


def _oracle_mu(k):
    return oracle.k_smooth_mean(k.float().numpy())["mean"].astype(np.float32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("smooth", [True, False])
def test_quantised_codes_and_scales_bit_exact(smooth, d):
    q, k, v = _inputs(2, 300, 200, 4, 2, d, 500 + d)
    mu = _oracle_mu(k) if smooth else None
    _, _, quant, pad = _fp8_call(q, k, v, mu, causal=False)
    ref_in = {"q": q.float().numpy(), "k": oracle.fp8.smooth_k(k.float().numpy(), mu), "v": v.float().numpy()}
    for name in ("q", "k", "v"):
        codes_ref, scales_ref, _ = oracle.quantize_blocks(ref_in[name])
        codes_gpu, scales_gpu = quant[name]
        np.testing.assert_array_equal(scales_gpu, scales_ref, err_msg=f"{name} scales")
        mism = int((codes_gpu != codes_ref).sum())
        assert mism == 0, f"{name}: {mism} of {codes_ref.size} E4M3 codes differ"
    assert (pad["q"] == 0).all() and (pad["k"] == 0).all(), "token padding must be zero codes"


def test_quantised_codes_bit_exact_at_tiny_magnitudes():
    # Heads scaled by powers of two (exact in bf16) move the block scales across the
    # quantiser's two division paths: the corrected reciprocal product for scales of at least
    # 2^-90 (head 1: scales near 2^-87, with elements small enough for the residual to
    # underflow) and the plain division below (head 2: scales near 2^-107).  Head 0 is the
    # usual N(0, 1) case.  Codes and scales must match the oracle's IEEE quotient bit for bit.
    q, k, v = _inputs(1, 260, 260, 3, 3, 128, 540, bias_std=0.0)
    factors = torch.tensor([1.0, 2.0 ** -80, 2.0 ** -100])
    q, k, v = (t.float() * factors[None, None, :, None] for t in (q, k, v))
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    _, _, quant, _ = _fp8_call(q, k, v, None, causal=False)
    for name, x in (("q", q), ("k", k), ("v", v)):
        codes_ref, scales_ref, _ = oracle.quantize_blocks(x.float().numpy())
        codes_gpu, scales_gpu = quant[name]
        assert scales_ref[0, 1].max() >= 2.0 ** -90 > scales_ref[0, 2].max(), "inputs must span both paths"
        np.testing.assert_array_equal(scales_gpu, scales_ref, err_msg=f"{name} scales")
        mism = int((codes_gpu != codes_ref).sum())
        assert mism == 0, f"{name}: {mism} of {codes_ref.size} E4M3 codes differ"


def _check_attention(q, k, v, mu, causal, what, heads=None, rows=None):
    o, lse, _, _ = _fp8_call(q, k, v, mu, causal)
    d = q.shape[3]
    o_ref, lse_ref, _ = oracle.fp8_attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                     mu=mu, scale=d ** -0.5, causal=causal, heads=heads,
                                                     rows=rows)
    o_g = o.float().numpy().astype(np.float64)
    l_g = lse.numpy().astype(np.float64)
    if heads is not None:
        o_g, l_g = o_g[:, :, heads], l_g[:, heads]
    if rows is not None:
        o_g, l_g = o_g[:, rows], l_g[:, :, rows]
    exact, _ = oracle.attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                        scale=d ** -0.5, causal=causal, heads=heads, rows=rows)
    print(f"[fp8] {what}: rel_l2 vs the unquantised oracle {_rel_l2(o_g, exact):.3e} (information only)", flush=True)
    rel, _, _ = assert_fp8_parity(o_g, o_ref, l_g, lse_ref, what)
    return rel


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_gqa(causal, d):
    q, k, v = _inputs(2, 300, 200, 4, 2, d, 600 + d)
    _check_attention(q, k, v, _oracle_mu(k), causal, f"ragged gqa d{d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", [(700, 520), (520, 700), (900, 900)], ids=["q700k520", "q520k700", "q900k900"])
def test_causal_pairs_ragged(shape, d):
    # causal grids with 5 to 8 query blocks, paired (n-1-j, j) with a middle block left over when
    # n is odd, ragged last blocks, and more or fewer keys than queries
    sq, sk = shape
    q, k, v = _inputs(1, sq, sk, 2, 1, d, 900 + d + sq)
    _check_attention(q, k, v, _oracle_mu(k), True, f"causal pairs d{d} {sq}x{sk}")


@pytest.mark.parametrize("sq, sk", [(300, 333), (640, 200)])
def test_two_blocks_per_workgroup(sq, sk):
    # non-causal d128 grids that still fill the device with two query blocks per workgroup (256
    # heads) take the packed kernel; an odd block count leaves the last workgroup's second block
    # empty (no rows to store)
    q, k, v = _inputs(1, sq, sk, 256, 256, 128, 950 + sq)
    _check_attention(q, k, v, _oracle_mu(k), False, f"two blocks per workgroup {sq}x{sk}",
                     heads=[0, 1, 100, 255])


def test_no_smoothing():
    q, k, v = _inputs(1, 256, 384, 2, 2, 128, 700, bias_std=0.0)
    _check_attention(q, k, v, None, False, "no smoothing")


def test_full_fp8_workload_sampled_heads():
    w = workloads.WORKLOADS["fp8_ksmooth_d128"]
    q, k, v = workloads.make_qkv(w)
    mu = _oracle_mu(k)
    _check_attention(q, k, v, mu, w.causal, "fp8 workload", heads=[0, 7, 15])


def test_full_fp8_workload_causal_sampled_heads():
    # The same inputs under the causal mask: 32 query blocks per head run as 16 workgroups that
    # each take blocks n-1-j and j; every row of three heads, i.e. every pair of those heads
    w = workloads.WORKLOADS["fp8_ksmooth_d128"]
    q, k, v = workloads.make_qkv(w)
    mu = _oracle_mu(k)
    _check_attention(q, k, v, mu, True, "fp8 workload causal", heads=[0, 7, 15])


def test_long_context_fp8_sampled():
    # b1 h5 65536^2: 512 K/V scale blocks per head; sampled rows of the first and last head
    w = workloads.WORKLOADS["fp8_long_h5"]
    q, k, v = workloads.make_qkv(w)
    mu = _oracle_mu(k)
    rows = workloads.sample_indices(w.sq, 96, 13, include=[0, 127, 128, w.sq // 2, w.sq - 1])
    _check_attention(q, k, v, mu, w.causal, "fp8 long context", heads=[0, 4], rows=rows)


def test_gpu_gate_then_fp8_matches_oracle_pipeline():
    # The whole quantised call: GPU gate -> GPU fp8 attention, against oracle gate -> oracle fp8.
    import head_attention_forward_flash_amd as mha
    dev = require_gpu()
    q, k, v = _inputs(1, 512, 512, 4, 4, 128, 800)
    kd = k.to(dev)
    mean, gate = mha.k_smooth_mean(kd)
    o, lse, _ = mha.mha_fwd_fp8(q.to(dev), kd, v.to(dev), k_mean=mean)
    torch.cuda.synchronize()
    mu_ref = _oracle_mu(k)
    assert gate.cpu().numpy().all()
    o_ref, lse_ref, _ = oracle.fp8_attention_forward(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                                     mu=mu_ref, scale=128 ** -0.5, causal=False)
    assert_fp8_parity(o.cpu().float().numpy().astype(np.float64), o_ref, lse.cpu().numpy().astype(np.float64),
                      lse_ref, "gate+fp8 pipeline")


def test_fp8_deterministic():
    q, k, v = _inputs(1, 400, 400, 2, 2, 128, 900)
    mu = _oracle_mu(k)
    a = _fp8_call(q, k, v, mu, True)
    b = _fp8_call(q, k, v, mu, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("q0", [4.0, 64.0])
def test_running_max_rising_in_steps(q0):
    # Queries point along channel 0 (q0) and key j carries j / 8 there, so each row's scores
    # climb along the keys by q0 * 4 / sqrt(128) * log2(e) per 32-key block: about 2 for q0 = 4
    # (below the rescale threshold) and about 33 for q0 = 64 (a rescale every block).
    d, sq, sk = 128, 256, 384
    q = workloads.make_random((1, sq, 2, d), 7100, dtype=torch.float32, std=0.05)
    k = workloads.make_random((1, sk, 2, d), 7101, dtype=torch.float32, std=0.05)
    q[..., 0] = q0
    k[0, :, :, 0] = (torch.arange(sk, dtype=torch.float32) / 8.0)[:, None]
    v = workloads.make_random((1, sk, 2, d), 7102)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    for causal in (False, True):
        _check_attention(q, k, v, _oracle_mu(k), causal, f"ramp q0={q0} causal={causal}")


def test_late_score_spike_overflows_the_reference():
    # As the bf16 test of the same name: one late key scores ~150 above the rest, so the fp8
    # kernel's speculative exponentials overflow and the block takes a new reference.
    d, s = 128, 384
    q = workloads.make_random((1, s, 2, d), 8200, dtype=torch.float32, std=0.1)
    k = workloads.make_random((1, s, 2, d), 8201, dtype=torch.float32, std=0.1)
    q[..., 0] = 1.0
    k[0, 300, :, 0] = 150.0 * d ** 0.5
    v = workloads.make_random((1, s, 2, d), 8202)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    for causal in (False, True):
        _check_attention(q, k, v, None, causal, f"spike causal={causal}")
