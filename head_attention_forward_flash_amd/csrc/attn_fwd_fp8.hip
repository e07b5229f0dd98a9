// Attention forward on E4M3-quantised, K-smoothed inputs (d = 128), gfx950.
//
// The attention side of the FP8 hd128 mha_v4 recipe ("[HIP] Mha v4: run the
// K-smoothing gate as one HIP call", Performance table; "MHA v4: fixes,
// refactor, new kernel, perf tweaks", BF16/FP8 recipe).  Inputs are the codes
// and per-(batch, head, 128-token block) fp32 scales written by quant_fp8.
//
// Same decomposition as the bf16 kernel (4 waves x 32 query rows, 64-key
// tiles, one query per lane in S^T), with:
//   S^T = K8 Q8^T  on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulate),
//                  two k-steps of 64 channels; both operands read 32 bytes of
//                  their row per lane, so the MFMA's channel order cancels out;
//   scores         t = s * (scale_q * scale_k * softmax_scale * log2 e): one
//                  factor per tile, since a 64-key tile sits inside one
//                  128-token scale block and the 128 query rows are one block;
//   P.V            on bf16 MFMA: V codes are widened exactly to bf16 while the
//                  tile is staged (transposed) into LDS, and the V block scale is
//                  folded into P before P is rounded to bf16;
//   l, m, O        as in the bf16 kernel (l sums the unscaled probabilities).

#include "device_common.h"
#include "kernels.h"

namespace mha {
namespace {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int D = 128;
constexpr int NTHREADS = 256;
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ u32x2 buffer_load_b64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

// 4 E4M3 codes (one dword) -> 4 bf16 values in two dwords (exact widening).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    return u32x2{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(hi[0], hi[1])};
}

template <bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2) void attn_fwd_fp8_kernel(const Fp8AttnParams p) {
    constexpr int KROW = D + 16;          // bytes per K8 row in LDS
    constexpr int VROW = BN + 4;          // bf16 elements per V^T row in LDS
    constexpr int CBLK = D / 32;
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[BN * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * VROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;

    const int nwg = gridDim.x;
    const int nwg8 = nwg & ~7;
    const int pid = blockIdx.x;
    const int lid = pid < nwg8 ? (pid & 7) * (nwg8 >> 3) + (pid >> 3) : pid;
    const int mrev = lid % p.n_mblocks;
    const int bh = lid / p.n_mblocks;
    const int mblk = CAUSAL ? (p.n_mblocks - 1 - mrev) : mrev;
    const int h = bh % p.hq;
    const int bb = bh / p.hq;
    const int g = h / p.group;
    const int bg = bb * p.hk + g;

    const uint32_t qslice = static_cast<uint32_t>(p.nq) * BM * D;
    const uint32_t kslice = static_cast<uint32_t>(p.nk) * BM * D;
    const auto qrs = make_rsrc(p.q + static_cast<int64_t>(bh) * qslice, qslice);
    const auto krs = make_rsrc(p.k + static_cast<int64_t>(bg) * kslice, kslice);
    const auto vrs = make_rsrc(p.v + static_cast<int64_t>(bg) * kslice, kslice);
    const float q_scale = p.q_scale[static_cast<int64_t>(bh) * p.nq + mblk];
    const float* k_scale = p.k_scale + static_cast<int64_t>(bg) * p.nk;
    const float* v_scale = p.v_scale + static_cast<int64_t>(bg) * p.nk;

    const int wave_row0 = mblk * BM + wave * 32;
    const int my_row = wave_row0 + col;

    // Q8 fragment: two k-steps of 64 channels, 32 codes per lane each
    i32x8 qf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const uint32_t off = static_cast<uint32_t>(my_row * D + ks * 64 + half * 32);
        const u32x4 a = buffer_load_b128(qrs, off);
        const u32x4 b = buffer_load_b128(qrs, off + 16);
        qf[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }

    const int kv_end = CAUSAL ? min(p.sk, (mblk + 1) * BM) : p.sk;
    const int ntiles = (kv_end + BN - 1) / BN;

    u32x4 kreg[2];
    u32x2 vreg[4];
    const int vkg = tid % 16;   // 4 keys
    const int vcg = tid / 16;   // 8 channels

    auto load_tile = [&](int t) {
        const int key0 = t * BN;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + NTHREADS * i;
            const int row = c / (D / 16);
            const int ch = c % (D / 16);
            kreg[i] = buffer_load_b128(krs, static_cast<uint32_t>((key0 + row) * D + ch * 16));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vreg[i] = buffer_load_b64(vrs, static_cast<uint32_t>((key0 + vkg * 4 + i) * D + vcg * 8));
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + NTHREADS * i;
            const int row = c / (D / 16);
            const int ch = c % (D / 16);
            *reinterpret_cast<u32x4*>(&k_lds[row * KROW + ch * 16]) = kreg[i];
        }
        // widen the 4 keys x 8 channels of V codes to bf16, then write channel rows
        u32x4 wide[4];   // per key: 8 bf16 = 4 dwords (channel pairs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x2 a = e4m3x4_to_bf16x4(vreg[i][0]);
            const u32x2 b = e4m3x4_to_bf16x4(vreg[i][1]);
            wide[i] = u32x4{a[0], a[1], b[0], b[1]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int dw = e >> 1;
            const bool hi = e & 1;
            uint32_t w[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t a = wide[2 * i][dw];
                const uint32_t c2 = wide[2 * i + 1][dw];
                w[i] = hi ? ((a >> 16) | (c2 & 0xffff0000u)) : ((a & 0xffffu) | (c2 << 16));
            }
            *reinterpret_cast<u32x2*>(&v_lds[(vcg * 8 + e) * VROW + vkg * 4]) = u32x2{w[0], w[1]};
        }
    };

    f32x16 oacc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
    float m_run = kNegInf;
    float l_run = 0.f;

    if (ntiles > 0) load_tile(0);

    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1);

        const int kblk = (t * BN) / BM;
        const float c = q_scale * k_scale[kblk] * p.scale_log2;
        const float sv = v_scale[kblk];

        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
            const uint8_t* krow = &k_lds[(kb * 32 + col) * KROW + half * 32];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(krow + ks * 64);
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(krow + ks * 64 + 16);
                const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                      (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[kb], 0, 0, 0, 0, 0, 0);
            }
        }

        const int key0 = t * BN;
        const bool need_mask = (key0 + BN > p.sk) || (CAUSAL && key0 + BN - 1 > wave_row0);
        float mt = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float x = s[kb][j] * c;
                if (need_mask) {
                    const int key = key0 + kb * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
                    if (key >= p.sk || (CAUSAL && key > my_row)) x = kNegInf;
                }
                s[kb][j] = x;
                mt = fmaxf(mt, x);
            }
        }
        mt = fmaxf(mt, swap_halves(mt));

        const float m_new = fmaxf(m_run, mt);
        if (__any(m_new > m_run + kRescaleThreshold)) {
            const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == kNegInf) ? 0.f : m_run;

        bf16x8 pf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = fast_exp2(s[ks >> 1][(ks & 1) * 8 + 2 * i] - m_use);
                const float p1 = fast_exp2(s[ks >> 1][(ks & 1) * 8 + 2 * i + 1] - m_use);
                l_run += p0 + p1;
                w[i] = pack_bf16x2(p0 * sv, p1 * sv);
            }
            pf[ks] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }

#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) {
            const uint16_t* vrow = &v_lds[(cb * 32 + col) * VROW + half * 4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + ks * 16);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + ks * 16 + 8);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], oacc[cb], 0, 0, 0);
            }
        }
    }

    const float l_tot = l_run + swap_halves(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (my_row < p.sq) {
        uint16_t* orow = static_cast<uint16_t*>(p.o) + (bb * p.ov.sb + h * p.ov.sh + my_row * p.ov.ss);
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int ch = cb * 32 + grp * 8 + half * 4;
                const uint32_t w0 = pack_bf16x2(oacc[cb][grp * 4 + 0] * inv, oacc[cb][grp * 4 + 1] * inv);
                const uint32_t w1 = pack_bf16x2(oacc[cb][grp * 4 + 2] * inv, oacc[cb][grp * 4 + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + ch) = u32x2{w0, w1};
            }
        }
        if (p.lse != nullptr && half == 0) {
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
            p.lse[(static_cast<int64_t>(bb) * p.hq + h) * p.sq + my_row] = lse;
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const Fp8AttnParams& p, int d, bool causal, hipStream_t stream) {
    if (d != D) return hipErrorInvalidValue;
    const int64_t nwg = static_cast<int64_t>(p.b) * p.hq * p.n_mblocks;
    if (nwg == 0) return hipSuccess;
    if (causal)
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<true>), dim3(static_cast<unsigned>(nwg)), dim3(NTHREADS), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((attn_fwd_fp8_kernel<false>), dim3(static_cast<unsigned>(nwg)), dim3(NTHREADS), 0,
                           stream, p);
    return hipGetLastError();
}

}  // namespace mha
