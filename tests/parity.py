"""Helpers shared by the GPU parity tests: device checks, oracle calls per head, metrics."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle

# Tolerances for the bf16 path (float64 oracle as the reference).
BF16_MAX_ABS = 1e-2          # per element, plus the bf16 output rounding allowance below
BF16_ROUND_ALLOWANCE = 2.0 ** -8   # |O| * 2^-8 = one bf16 ulp at |O|: O is stored in bf16
BF16_REL_L2 = 5e-3
# The kernels sum the bf16-rounded probabilities that enter P.V (relative error <= 2^-9
# each), so ln(l) can be off by up to ~2^-9 on rows with few keys; 2^-8 leaves room for the
# fp32 score rounding on top.
LSE_MAX_ABS = 2.0 ** -8
FP8_REL_L2 = 2e-2


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
    excess = float((diff - (BF16_MAX_ABS + BF16_ROUND_ALLOWANCE * np.abs(o_ref))).max()) if diff.size else -1.0
    denom = float(np.linalg.norm(o_ref))
    rel_l2 = float(np.linalg.norm(o_gpu - o_ref) / denom) if denom > 0 else float(np.linalg.norm(o_gpu - o_ref))
    return {"max_abs": max_abs, "excess": excess, "rel_l2": rel_l2}


def assert_bf16_parity(o_gpu, o_ref, lse_gpu=None, lse_ref=None, what=""):
    m = bf16_metrics(o_gpu, o_ref)
    print(f"[parity] {what}: max_abs={m['max_abs']:.3e} rel_l2={m['rel_l2']:.3e}", flush=True)
    assert m["excess"] <= 0.0, f"{what}: max-abs {m['max_abs']:.4e} exceeds 1e-2 + 2^-8|O| ({m})"
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
