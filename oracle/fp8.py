"""FP8 (E4M3) block quantisation and quantised-attention oracle.  Test infrastructure only.

Sources: "[HIP] Mha v4: run the K-smoothing gate as one HIP call" (ROCm aiter
PR 7754), Summary and Performance table: the quantised mha_v4 call with an
FP8 hd128 recipe, whose K is smoothed by the per-head K mean; "MHA v4: fixes,
refactor, new kernel, perf tweaks" (ROCm aiter PR 5335), Motivation and
Kernels list: BF16/FP8 recipes of that op.  The pages name the recipe but not
its rounding rules, so the readings taken here are:

  * format: OCP E4M3 "fn" (bias 7, 3 mantissa bits, subnormals, largest
    finite 448, no infinities), round to nearest even, saturating at +-448;
  * scales: one float32 scale per (batch, head, block of 128 tokens), over all
    channels of the block; scale = amax / 448 rounded to float32
    (1.0 when amax == 0);
  * codes: q = E4M3(float32(x / scale)), the division done in float32;
  * K smoothing: x_K = float32(float32(K) - mu) with mu the float32 per-(batch,
    kv head, channel) mean, subtracted before quantising; Q and V are quantised
    from float32(Q), float32(V);
  * attention runs, in float64, on the dequantised values q * scale, with the
    same softmax scale, causal mask and head mapping as the bf16 path.

Everything returned as "values" is float64; the arithmetic the quantiser
performs in float32 is emulated with numpy float32 operations, which are
IEEE-754 correctly rounded.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6      # smallest normal: 2^-6
E4M3_MANT_BITS = 3
E4M3_BIAS = 7
BLOCK_TOKENS = 128


def e4m3_round(x) -> np.ndarray:
    """Round float values to the nearest E4M3 value (ties to even), saturating at +-448.

    The spacing of E4M3 values in [2^e, 2^(e+1)) is 2^(e-3) for e >= -6 and
    2^-9 below 2^-6 (subnormals).  Dividing by that power-of-two spacing is
    exact in float64, so rint (ties to even) on the quotient rounds exactly.
    Zero keeps its sign.  NaN inputs stay NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, exp2 = np.frexp(mag)                   # mag = f * 2^exp2, f in [0.5, 1)
    e = exp2.astype(np.int64) - 1             # floor(log2(mag)) for mag > 0
    e = np.maximum(e, E4M3_MIN_NORMAL_EXP)    # subnormals share the 2^-9 spacing
    quantum = np.ldexp(1.0, e - E4M3_MANT_BITS)
    r = np.rint(mag / quantum) * quantum
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def e4m3_encode(values) -> np.ndarray:
    """Bit pattern (uint8) of E4M3 values (inputs must already lie on the E4M3 grid)."""
    v = np.asarray(values, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    mag = np.abs(v)
    codes = np.zeros(v.shape, dtype=np.uint8)
    normal = mag >= 2.0 ** E4M3_MIN_NORMAL_EXP
    sub = (mag > 0) & ~normal
    _, exp2 = np.frexp(np.where(normal, mag, 1.0))
    e = exp2.astype(np.int64) - 1
    mant = np.where(normal, mag / np.ldexp(1.0, e) * 8.0 - 8.0, 0.0)
    field = np.where(normal, e + E4M3_BIAS, 0)
    sub_mant = np.where(sub, mag / 2.0 ** -9, 0.0)
    mant_all = np.where(normal, mant, sub_mant)
    if np.any(mant_all != np.floor(mant_all)) or np.any(mag > E4M3_MAX):
        raise ValueError("value not on the E4M3 grid")
    codes = (field.astype(np.uint8) << 3) | mant_all.astype(np.uint8)
    codes = codes | sign
    codes = np.where(np.isnan(v), np.uint8(0x7F), codes).astype(np.uint8)
    return codes


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of E4M3 bit patterns (0x7F / 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    field = (c >> 3) & 0xF
    mant = c & 0x7
    val = np.where(field == 0,
                   mant * 2.0 ** -9,
                   (1.0 + mant / 8.0) * np.ldexp(1.0, field - E4M3_BIAS))
    val = sign * val
    return np.where((field == 15) & (mant == 7), np.nan, val)


def quantize_blocks(x_f32, block: int = BLOCK_TOKENS):
    """Quantise a float32 [b, s, h, d] tensor per (b, h, block of tokens).

    Returns (codes uint8 [b, s, h, d], scales float32 [b, h, nblk], values float64
    [b, s, h, d]) where values = decode(codes) * scale of the element's block.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    b, s, h, d = x.shape
    nblk = (s + block - 1) // block
    codes = np.zeros((b, s, h, d), dtype=np.uint8)
    scales = np.ones((b, h, nblk), dtype=np.float32)
    values = np.zeros((b, s, h, d), dtype=np.float64)
    for bi in range(b):
        for hi in range(h):
            for blk in range(nblk):
                t0, t1 = blk * block, min(s, (blk + 1) * block)
                xb = x[bi, t0:t1, hi, :]                                # float32
                amax = np.float32(np.max(np.abs(xb))) if xb.size else np.float32(0)
                scale = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))
                scaled = (xb / scale).astype(np.float32)               # float32 division
                qv = e4m3_round(scaled)
                codes[bi, t0:t1, hi, :] = e4m3_encode(qv)
                scales[bi, hi, blk] = scale
                values[bi, t0:t1, hi, :] = qv * np.float64(scale)
    return codes, scales, values


def smooth_k(k, mu):
    """x_K = float32(float32(K) - mu) with mu [b, hk, d] float32 (None: no smoothing)."""
    k32 = np.asarray(k, dtype=np.float32)
    if mu is None:
        return k32
    mu32 = np.asarray(mu, dtype=np.float32)
    return (k32 - mu32[:, None, :, :]).astype(np.float32)


def fp8_attention_forward(q, k, v, *, mu=None, scale, causal, heads=None, rows=None, batches=None):
    """Quantise Q, K - mu and V to E4M3 blocks, then run float64 attention on the dequantised values.

    Returns (o, lse, quant) where quant holds the (codes, scales) of q, k, v.
    """
    q32 = np.asarray(q, dtype=np.float32)
    v32 = np.asarray(v, dtype=np.float32)
    k32 = smooth_k(k, mu)
    qc, qs, qv = quantize_blocks(q32)
    kc, ks, kv = quantize_blocks(k32)
    vc, vs, vv = quantize_blocks(v32)
    o, lse = attention_forward(qv, kv, vv, scale=scale, causal=causal, heads=heads, rows=rows,
                               batches=batches)
    quant = {"q": (qc, qs), "k": (kc, ks), "v": (vc, vs)}
    return o, lse, quant
