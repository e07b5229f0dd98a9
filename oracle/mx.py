"""MXFP8 (E4M3 elements, E8M0 block exponents) quantisation and attention oracle.  Test infrastructure only.

Sources: "[HIP] Mha v4: run the K-smoothing gate as one HIP call" (ROCm aiter
PR 7754), commit message table: an "MXFP8 hd128" recipe of the quantised
mha_v4 call next to the FP8 one, sharing its K-smoothing gate; "MHA v4: fixes,
refactor, new kernel, perf tweaks" (ROCm aiter PR 5335), suppressed review
comments: MX descales are uint8 E8M0 values, one per 1x32 block.  The pages
name the recipe and the scale format but not the quantiser, so the readings
taken here follow the OCP Microscaling (MX) v1.0 format definition:

  * a block is 32 consecutive elements along the head dimension (the
    contiguous axis of [b, s, h, d]; the contraction axis of Q K^T), for Q,
    K - mean and V alike;
  * the block's shared exponent is E = floor(log2(amax)) - 8, 8 being the
    exponent of E4M3's largest normal (448 = 1.75 * 2^8), clamped to
    [-127, 127]; it is stored as the E8M0 byte E + 127; an all-zero block
    stores byte 0;
  * element code = E4M3(x / 2^E): round to nearest even, saturating at +-448
    (x / 2^E can reach up to 2^9, past E4M3's range);
  * the dequantised value is decode(code) * 2^E;
  * K smoothing and the float32 inputs are those of the FP8 recipe
    (``fp8.smooth_k``); attention runs in float64 on the dequantised values.

Everything returned as "values" is float64.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward
from .fp8 import e4m3_decode, e4m3_encode, e4m3_round, smooth_k

MX_BLOCK = 32
E4M3_EMAX = 8          # 448 = 1.75 * 2^8
E8M0_BIAS = 127


def mx_quantize(x_f32):
    """MXFP8-quantise a float32 tensor along its last axis (a multiple of 32).

    Returns (codes uint8 [..., d], exps uint8 [..., d/32] (E8M0 bytes), values
    float64 [..., d]).
    """
    x = np.asarray(x_f32, dtype=np.float32).astype(np.float64)
    d = x.shape[-1]
    if d % MX_BLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))          # amax = f * 2^e2, f in [0.5, 1)
    shared = (e2.astype(np.int64) - 1) - E4M3_EMAX           # floor(log2(amax)) - emax
    shared = np.clip(shared, -E8M0_BIAS, E8M0_BIAS)
    exps = np.where(amax > 0, shared + E8M0_BIAS, 0).astype(np.uint8)
    scale = np.ldexp(1.0, exps.astype(np.int64) - E8M0_BIAS)[..., None]
    q = e4m3_round(blocks / scale)                           # exact power-of-two division
    codes = e4m3_encode(q).reshape(x.shape)
    values = (e4m3_decode(codes).reshape(blocks.shape) * scale).reshape(x.shape)
    return codes, exps, values


def mx_dequantize(codes, exps):
    """float64 values of MXFP8 codes [..., d] with E8M0 block bytes [..., d/32]."""
    c = np.asarray(codes, dtype=np.uint8)
    d = c.shape[-1]
    scale = np.ldexp(1.0, np.asarray(exps, dtype=np.int64) - E8M0_BIAS)
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (d // MX_BLOCK, MX_BLOCK)) * scale[..., None]
    return vals.reshape(c.shape)


def mxfp8_attention_forward(q, k, v, *, mu=None, scale, causal, heads=None, rows=None, batches=None):
    """MXFP8-quantise Q, K - mu and V, then run float64 attention on the dequantised values.

    Returns (o, lse, quant) where quant holds the (codes, exps) of q, k, v.
    """
    qc, qe, qv = mx_quantize(np.asarray(q, dtype=np.float32))
    kc, ke, kv = mx_quantize(smooth_k(k, mu))
    vc, ve, vv = mx_quantize(np.asarray(v, dtype=np.float32))
    o, lse = attention_forward(qv, kv, vv, scale=scale, causal=causal, heads=heads, rows=rows,
                               batches=batches)
    return o, lse, {"q": (qc, qe), "k": (kc, ke), "v": (vc, ve)}
