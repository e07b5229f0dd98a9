// FP8 (OCP E4M3) block quantisation of Q, K - mean and V for the quantised
// attention call: the producer side of the FP8 hd128 mha_v4 recipe of
// "[HIP] Mha v4: run the K-smoothing gate as one HIP call" (Summary: K is
// smoothed by its per-head mean before quantisation; Performance table: FP8
// hd128) and "MHA v4: fixes, refactor, new kernel, perf tweaks" (BF16/FP8
// recipe, quantisation producers).
//
// One workgroup per (tensor, batch, block of 128 tokens, head):
//   x      = fp32(bf16 input)                 (K: fp32(K) - mean[b, h, c], one fp32 rounding)
//   amax   = max |x| over the block's tokens and channels (wave max, then LDS)
//   scale  = amax / 448 in fp32 (1 when amax == 0)
//   code   = E4M3(x / scale): the correctly rounded fp32 quotient (one reciprocal per
//            thread and a corrected product per element), clamp to +-448 (a no-op
//            except for the last half-ulp above 448, which rounds to 448 anyway), then
//            v_cvt_pk_fp8_f32 (round to nearest even)
// Codes go to a token-padded [b, h, nblk*128, D] array (tokens past s are
// written as zero codes), scales to [b, h, nblk].  For V the codes' values are
// stored widened to bf16 instead (E4M3 values are exactly representable), which
// is the form the P.V MFMA consumes.  HBM-bound: 2 bytes read and 1 byte (V: 2)
// written per element.
//
// MXFP8 (the MXFP8 hd128 recipe of the first page's commit message table, with
// the uint8 E8M0 per-1x32 descales of the second page's review comments; block
// format of OCP Microscaling v1.0): instead of one fp32 scale per 128 tokens,
// every 32 channels of a token row share an exponent
//   E      = clamp(floor(log2(amax)) - 8, -127, 127), read from amax's exponent
//            field (8 = exponent of E4M3's largest normal, 448 = 1.75 * 2^8);
//            rows of zeros (and subnormal amax) take E = -127, byte 0
//   code   = E4M3(x * 2^-E), the product exact, saturated at +-448
// stored as the byte E + 127 in [b, h, nblk*128, D/32].  V is stored as
// decode(code) * 2^E in bf16 (exact while it stays in bf16's normal range),
// so the attention kernel needs no V scale at all.

#include "device_common.h"
#include "kernels.h"

namespace mha {
namespace {

constexpr int NT = 256;
constexpr int TOK = 128;

// MXFP8: every thread holds 8 channels of PASSES token rows; the 4 threads of a 32-channel
// block are adjacent lanes, so the block max takes two lane exchanges.
template <int D, int PASSES>
__device__ __forceinline__ void quant_rows_mx(const QuantParams& p, const float (&x)[PASSES][8], int bh, int blk,
                                              int r0, int c0) {
    constexpr int ROWS = TOK / PASSES;
    const int64_t row0 = static_cast<int64_t>(bh) * p.nblk * TOK + blk * TOK;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[ps][i]));
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        const int field = static_cast<int>(__float_as_uint(m) >> 23);     // m >= 0: no sign bit
        const int e = field == 0 ? -127 : max(field - 127 - 8, -127);     // at most 254 - 135 = 119
        const float inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);   // 2^-e, normal
        const float up = e > -127 ? __uint_as_float(static_cast<uint32_t>(127 + e) << 23) : 0x1p-127f;
        uint32_t packed[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(x[ps][half * 4 + j] * inv, -448.f), 448.f);
            int wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], wv, true);
            packed[half] = static_cast<uint32_t>(wv);
        }
        const int64_t row = row0 + ps * ROWS + r0;
        if (p.widen) {
            // decode(code) * 2^e, exact in fp32 and (in bf16's normal range) in bf16
            uint32_t wide[4];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(packed[half]), false);
                const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(packed[half]), true);
                wide[2 * half] = pack_bf16x2(lo[0] * up, lo[1] * up);
                wide[2 * half + 1] = pack_bf16x2(hi[0] * up, hi[1] * up);
            }
            *reinterpret_cast<u32x4*>(p.codes + (row * D + c0) * 2) = u32x4{wide[0], wide[1], wide[2], wide[3]};
        } else {
            *reinterpret_cast<u32x2*>(p.codes + row * D + c0) = u32x2{packed[0], packed[1]};
        }
        if (p.exps != nullptr && (c0 & 31) == 0)
            p.exps[row * (D / 32) + c0 / 32] = static_cast<uint8_t>(e + 127);
    }
}

// Workgroup ids run over heads fastest, then token blocks, then batches: workgroups that are
// dispatched together read neighbouring 2*D-byte pieces of the same BSHD token rows.
template <int D>
__device__ __forceinline__ void quant_block(const QuantParams& p, int id, float* red) {
    constexpr int TPR = D / 8;          // threads per token row (16 B each)
    constexpr int ROWS = NT / TPR;      // token rows per pass
    constexpr int PASSES = TOK / ROWS;
    const int h = id % p.heads;
    const int blk = (id / p.heads) % p.nblk;
    const int bb = id / (p.heads * p.nblk);
    const int bh = bb * p.heads + h;
    const int tid = threadIdx.x;
    const int c0 = (tid % TPR) * 8;
    const int r0 = tid / TPR;

    const char* base = static_cast<const char*>(p.src) + 2 * (bb * p.sv.sb + h * p.sv.sh);
    const auto rs = make_rsrc(base, p.sv.slice_bytes);

    float mu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mu[i] = 0.f;
    if (p.mean != nullptr) {
        const float* m = p.mean + static_cast<int64_t>(bh) * D + c0;
#pragma unroll
        for (int i = 0; i < 8; ++i) mu[i] = m[i];
    }

    float x[PASSES][8];
    float amax = 0.f;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int tok = blk * TOK + ps * ROWS + r0;
        const uint32_t off = tok < p.s ? static_cast<uint32_t>((tok * p.sv.ss + c0) * 2) : kOutOfRange;
        const u32x4 w = buffer_load_b128(rs, off);
        const bool live = tok < p.s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = bf16_bits_to_float(w[i] & 0xffffu);
            const float hi = bf16_bits_to_float(w[i] >> 16);
            x[ps][2 * i] = live ? lo - mu[2 * i] : 0.f;
            x[ps][2 * i + 1] = live ? hi - mu[2 * i + 1] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[ps][i]));
    }
    if (p.mx) {
        quant_rows_mx<D, PASSES>(p, x, bh, blk, r0, c0);
        return;
    }
    // block max: within the wave, then across the 4 waves through LDS
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) amax = fmaxf(amax, __shfl_xor(amax, sh, 64));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax > 0.f ? amax / 448.0f : 1.0f)));

    // x / scale, correctly rounded, without a full division per element: with y = RN(1/scale),
    // q = RN(x y) is within an ulp of the quotient, r = x - q scale is exact in one FMA, and
    // RN(q + r y) is the correctly rounded quotient (Markstein's correction step; P. Markstein,
    // "IA-64 and Elementary Functions", the division theorems of its chapter on division).
    // r stays exact while |x| >= 2^-102; below that, with scale >= 2^-90, both quotients are
    // under 2^-12 and encode to the same (zero) code, their sign taken from x.  Blocks with a
    // smaller scale divide element by element.
    if (scale >= 0x1p-90f) {
        const float recip = 1.0f / scale;
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = x[ps][i];
                const float q = v * recip;
                const float r = fmaf(-q, scale, v);
                x[ps][i] = copysignf(fmaf(r, recip, q), v);
            }
        }
    } else {
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[ps][i] = x[ps][i] / scale;
        }
    }

    const int64_t elem0 = static_cast<int64_t>(bh) * p.nblk * TOK + blk * TOK;   // first row of the block
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        uint32_t packed[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(x[ps][half * 4 + j], -448.f), 448.f);
            int wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], wv, true);
            packed[half] = static_cast<uint32_t>(wv);
        }
        const int row = ps * ROWS + r0;
        if (p.widen) {
            // the codes' values, widened to bf16 (every E4M3 value is a bf16 value)
            uint32_t wide[4];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(packed[half]), false);
                const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(packed[half]), true);
                wide[2 * half] = pack_bf16x2(lo[0], lo[1]);
                wide[2 * half + 1] = pack_bf16x2(hi[0], hi[1]);
            }
            uint8_t* dst = p.codes + ((elem0 + row) * D + c0) * 2;
            *reinterpret_cast<u32x4*>(dst) = u32x4{wide[0], wide[1], wide[2], wide[3]};
        } else {
            *reinterpret_cast<u32x2*>(p.codes + (elem0 + row) * D + c0) = u32x2{packed[0], packed[1]};
        }
    }
    if (tid == 0) p.scales[static_cast<int64_t>(bh) * p.nblk + blk] = scale;
}

template <int D>
__global__ __launch_bounds__(NT) void quant_fp8_kernel(const QuantParams q, const QuantParams k,
                                                       const QuantParams v) {
    __shared__ float red[4];
    const int nq = q.b * q.heads * q.nblk;
    const int nk = k.b * k.heads * k.nblk;
    int id = blockIdx.x;
    if (id < nq) {
        quant_block<D>(q, id, red);
    } else if ((id -= nq) < nk) {
        quant_block<D>(k, id, red);
    } else {
        quant_block<D>(v, id - nk, red);
    }
}

}  // namespace

hipError_t launch_quant_fp8(const QuantParams& q, const QuantParams& k, const QuantParams& v, hipStream_t stream) {
    const int64_t total = int64_t(q.b) * q.heads * q.nblk + int64_t(k.b) * k.heads * k.nblk +
                          int64_t(v.b) * v.heads * v.nblk;
    if (total == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(total));
    if (q.d == 128)
        hipLaunchKernelGGL((quant_fp8_kernel<128>), grid, dim3(NT), 0, stream, q, k, v);
    else if (q.d == 64)
        hipLaunchKernelGGL((quant_fp8_kernel<64>), grid, dim3(NT), 0, stream, q, k, v);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mha
