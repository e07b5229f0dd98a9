"""Helpers shared by the GPU parity tests: device checks, oracle calls per head, metrics."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle

# Tolerances for the bf16 path (float64 oracle as the reference).
BF16_MAX_ABS = 1e-2          # per element, flat, wherever bf16 can hold O that closely
# O is stored in bf16, whose rounding alone costs up to half an ulp: at most 2^-9 |O| < 0.0078
# below |O| = 4, so there the flat 1e-2 bound is asserted as it stands.  From |O| = 4 on, half
# an ulp (0.0156 in [4, 8)) exceeds 1e-2 by itself; such elements may add one bf16 ulp, 2^-8 |O|.
BF16_FLAT_BELOW = 4.0
BF16_ROUND_ALLOWANCE = 2.0 ** -8
BF16_REL_L2 = 5e-3
# The kernels sum the bf16-rounded probabilities that enter P.V (relative error <= 2^-9
# each), so ln(l) can be off by up to ~2^-9 on rows with few keys; 2^-8 leaves room for the
# fp32 score rounding on top.
LSE_MAX_ABS = 2.0 ** -8
FP8_REL_L2 = 2e-2            # against the oracle that applies the same quantisation
# FP8 / MXFP8 LSE, per element: |LSE_gpu - LSE_ref| <= 2^-8 + 2^-14 |LSE_ref|.  The row sum adds
# the bf16-rounded P fed to P.V (relative error <= 2^-9 per term, as on the bf16 path); the
# V block scale enters P through exp2(... + log2 s_v) and leaves the sum through 1/s_v, both
# hardware-rounded (a few 2^-23 relative, and 2^-16 absolute in the exponent at most); fp32
# accumulation of the row sum over 2^16 keys stays within 2^-14 in the worst case.  2^-8
# covers these.  The scores grow with the inputs' magnitude, and the fp8 MFMA does not round
# its dot products as IEEE fp32 does: on scores of ~600 (in natural-log units) the LSE came
# out 1.1e-2 off, about 2^-16 of its magnitude, where fp32 rounding would give ~2^-22.
# 2^-14 |LSE| bounds that with a factor of 4 to spare.
FP8_LSE_ABS = 2.0 ** -8
FP8_LSE_REL = 2.0 ** -14


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    import head_attention_forward_flash_amd as mha
    mha.load_library()   # raises if the library is missing: no silent fallback
    return torch.device("cuda", 0)


def to_np(t: torch.Tensor) -> np.ndarray:
    """bfloat16/float tensor -> float64 numpy (bfloat16 widens exactly)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def oracle_heads(q, k, v, heads, rows, *, scale, causal, batch=0):
    """Oracle O [len(rows), len(heads), dv] and LSE [len(heads), len(rows)] for one batch.

    Each selected query head is evaluated as its own single-head problem with the kv head
    the grouped-query mapping assigns it (head h reads kv head h // (hq // hk)); heads are
    independent in the definition, so this equals evaluating the whole tensor.
    """
    hq, hk = q.shape[2], k.shape[2]
    grp = hq // hk
    outs, lses = [], []
    for h in heads:
        g = h // grp
        qh = q[batch:batch + 1, :, h:h + 1, :].float().numpy()
        kh = k[batch:batch + 1, :, g:g + 1, :].float().numpy()
        vh = v[batch:batch + 1, :, g:g + 1, :].float().numpy()
        o, l = oracle.attention_forward(qh, kh, vh, scale=scale, causal=causal, rows=rows)
        outs.append(o[0, :, 0, :])
        lses.append(l[0, 0, :])
    return np.stack(outs, axis=1), np.stack(lses, axis=0)


def bf16_metrics(o_gpu: np.ndarray, o_ref: np.ndarray):
    diff = np.abs(o_gpu - o_ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    mag = np.abs(o_ref)
    allowance = np.where(mag < BF16_FLAT_BELOW, 0.0, BF16_ROUND_ALLOWANCE * mag)
    excess = float((diff - (BF16_MAX_ABS + allowance)).max()) if diff.size else -1.0
    denom = float(np.linalg.norm(o_ref))
    rel_l2 = float(np.linalg.norm(o_gpu - o_ref) / denom) if denom > 0 else float(np.linalg.norm(o_gpu - o_ref))
    return {"max_abs": max_abs, "excess": excess, "rel_l2": rel_l2}


def assert_bf16_parity(o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    m = bf16_metrics(o_gpu, o_ref)
    print(f"[parity] {what}: max_abs={m['max_abs']:.3e} rel_l2={m['rel_l2']:.3e}", flush=True)
    assert m["excess"] <= 0.0, f"{what}: max-abs {m['max_abs']:.4e} exceeds 1e-2 (+ 2^-8|O| where |O| >= 4) ({m})"
    assert m["rel_l2"] <= BF16_REL_L2, f"{what}: rel-L2 {m['rel_l2']:.4e} > {BF16_REL_L2}"
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: LSE finiteness differs"
        if fin.any():
            err = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max())
            assert err <= LSE_MAX_ABS, f"{what}: LSE max-abs {err:.3e} > {LSE_MAX_ABS}"
        assert np.array_equal(lse_gpu[~fin], lse_ref[~fin]), f"{what}: non-finite LSE values differ"
    return m


def scale_for(d_qk: int) -> float:
    return 1.0 / math.sqrt(d_qk)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    denom = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b) / denom) if denom > 0 else float(np.linalg.norm(a - b))


def assert_fp8_parity(o_gpu, o_ref, lse_gpu, lse_ref, what=""):
    """FP8 / MXFP8 parity: rel-L2 of the whole checked subset and of every checked row (one
    query row of one head, over its d_v channels) <= FP8_REL_L2, and the LSE per element.

    o_*: [b, rows, heads, d_v]; lse_*: [b, heads, rows].  A row whose reference output is all
    zero must come out all zero.
    """
    rel = rel_l2(o_gpu, o_ref)
    diff = np.linalg.norm(o_gpu - o_ref, axis=-1)          # [b, rows, heads]
    ref = np.linalg.norm(o_ref, axis=-1)
    zero = ref == 0
    row_rel = np.where(zero, 0.0, diff / np.where(zero, 1.0, ref))
    worst = float(row_rel.max()) if row_rel.size else 0.0
    fin = np.isfinite(lse_ref)
    lerr = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    print(f"[fp8-parity] {what}: rel_l2={rel:.3e} worst row rel_l2={worst:.3e} lse max-abs={lerr:.3e}", flush=True)
    assert rel <= FP8_REL_L2, f"{what}: rel-L2 {rel:.4e} > {FP8_REL_L2}"
    if row_rel.size:
        idx = np.unravel_index(int(np.argmax(row_rel)), row_rel.shape)
        assert worst <= FP8_REL_L2, f"{what}: row (b, row, head) = {idx} has rel-L2 {worst:.4e} > {FP8_REL_L2}"
    assert np.all(diff[zero] == 0.0), f"{what}: rows with an all-zero reference output are not zero"
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: LSE finiteness differs"
    assert np.array_equal(lse_gpu[~fin], lse_ref[~fin]), f"{what}: non-finite LSE values differ"
    if fin.any():
        excess = np.abs(lse_gpu[fin] - lse_ref[fin]) - (FP8_LSE_ABS + FP8_LSE_REL * np.abs(lse_ref[fin]))
        assert float(excess.max()) <= 0.0, f"{what}: LSE max-abs {lerr:.3e} exceeds 2^-8 + 2^-14|LSE|"
    return rel, worst, lerr


def block_rows(sq: int, block: int, seed: int) -> list:
    """One seeded query row inside every block of `block` rows of [0, sq) (the last block may be partial)."""
    rng = np.random.default_rng(seed)
    return [start + int(rng.integers(0, min(block, sq - start))) for start in range(0, sq, block)]


def assert_every_block_row(q, k, v, o, lse, *, scale, causal, seed, what, block=128):
    """Compare one seeded row of every (batch, query head, block of `block` rows) with the oracle.

    Every workgroup of the bf16 kernel covers 128 or 256 rows of one (batch, head), so this
    checks the output of every workgroup of a full-size launch, whatever the id remapping and
    block pairing do.  q, k, v, o: CPU BSHD tensors; lse: CPU [b, hq, sq].
    """
    b, sq, hq, _ = q.shape
    grp = hq // k.shape[2]
    og, orf, lg, lrf = [], [], [], []
    for bb in range(b):
        for h in range(hq):
            g = h // grp
            rows = block_rows(sq, block, seed * 1_000_003 + bb * 4099 + h)
            o_ref, l_ref = oracle.attention_forward(q[bb:bb + 1, :, h:h + 1].float().numpy(),
                                                    k[bb:bb + 1, :, g:g + 1].float().numpy(),
                                                    v[bb:bb + 1, :, g:g + 1].float().numpy(),
                                                    scale=scale, causal=causal, rows=rows)
            orf.append(o_ref[0, :, 0, :])
            lrf.append(l_ref[0, 0, :])
            og.append(to_np(o[bb, rows, h]))
            lg.append(lse[bb, h, rows].numpy().astype(np.float64))
    return assert_bf16_parity(np.concatenate(og), np.concatenate(orf), np.concatenate(lg), np.concatenate(lrf),
                              f"{what}: one row per (batch, head, {block}-row block), {b * hq} heads")
