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
//   scores         t = s * (scale_q * scale_k * |softmax_scale| * log2 e): one
//                  factor per tile, since a 64-key tile sits inside one
//                  128-token scale block and the 128 query rows are one block;
//                  the factor and the running max fold into one FMA before exp2;
//   P.V            on bf16 MFMA: V codes are widened exactly to bf16 while the
//                  tile is staged (transposed) into LDS, and the V block scale
//                  enters P through the exponent (p' = exp2(t - m + log2 scale_v))
//                  before P is rounded to bf16;
//   l              sums the bf16 P' fed to P.V (v_dot2_f32_bf16), divided by the
//                  tile's V scale once per tile; two tiles of codes are in flight.

#include <type_traits>

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
    const float q_scale = p.q_scale[static_cast<int64_t>(bh) * p.nq + mblk];
    const float* k_scale = p.k_scale + static_cast<int64_t>(bg) * p.nk;
    const float* v_scale = p.v_scale + static_cast<int64_t>(bg) * p.nk;

    const int wave_row0 = mblk * BM + wave * 32;
    const int my_row = wave_row0 + col;

    // Q8 fragment: two k-steps of 64 channels, 32 codes per lane each.  softmax(c*s) with
    // c < 0 equals softmax(|c| * (-s)): a negative scale flips the sign bits of Q (exact).
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80808080u : 0u;
    i32x8 qf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const uint32_t off = static_cast<uint32_t>(my_row * D + ks * 64 + half * 32);
        const u32x4 a = buffer_load_b128(qrs, off) ^ qsign;
        const u32x4 b = buffer_load_b128(qrs, off + 16) ^ qsign;
        qf[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
    const float cq = q_scale * fabsf(p.scale_log2);   // base-2 factor of this block's scores, >= 0

    const int kv_end = CAUSAL ? min(p.sk, (mblk + 1) * BM) : p.sk;
    const int ntiles = (kv_end + BN - 1) / BN;

    // two tiles of codes in flight (loads of tile t+2 are issued while tile t is computed)
    constexpr int PF = 2;
    u32x4 kreg[PF][2];
    u32x2 vreg[PF][4];
    const int vkg = tid % 16;   // 4 keys
    const int vcg = tid / 16;   // 8 channels
    uint32_t koff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int chunk = tid + NTHREADS * i;
        koff[i] = static_cast<uint32_t>((chunk / (D / 16)) * D + (chunk % (D / 16)) * 16);
    }
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = static_cast<uint32_t>((vkg * 4 + i) * D + vcg * 8);

    auto load_tile = [&](int t, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        // tiles past the padded key range read nothing (empty buffer range)
        const uint32_t start = static_cast<uint32_t>(t) * BN * D;
        const uint32_t left = start < kslice ? kslice - start : 0u;
        const auto kr = make_rsrc(p.k + static_cast<int64_t>(bg) * kslice + (left ? start : 0), left);
        const auto vr = make_rsrc(p.v + static_cast<int64_t>(bg) * kslice + (left ? start : 0), left);
#pragma unroll
        for (int i = 0; i < 2; ++i) kreg[slot][i] = buffer_load_b128(kr, koff[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) vreg[slot][i] = buffer_load_b64(vr, voff[i]);
    };

    auto store_tile = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int chunk = tid + NTHREADS * i;
            *reinterpret_cast<u32x4*>(&k_lds[(chunk / (D / 16)) * KROW + (chunk % (D / 16)) * 16]) = kreg[slot][i];
        }
        // widen the 4 keys x 8 channels of V codes to bf16, then write channel rows
        u32x4 wide[4];   // per key: 8 bf16 = 4 dwords (channel pairs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x2 a = e4m3x4_to_bf16x4(vreg[slot][i][0]);
            const u32x2 b = e4m3x4_to_bf16x4(vreg[slot][i][1]);
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
    float m_run = kNegInf;   // running max in base-2 units of scaled scores
    float l_run = 0.f;

    auto compute_tile = [&](int t) __attribute__((always_inline)) {
        const int kblk = (t * BN) / BM;
        const float c = cq * k_scale[kblk];            // this tile's base-2 score factor
        const float log2_sv = __log2f(v_scale[kblk]);  // V block scale, folded into P
        const float inv_sv = 1.f / v_scale[kblk];

        // S^T = K8 Q8^T: two 32-key accumulators, two k-steps of 64 channels
        f32x16 s[2] = {f32x16{}, f32x16{}};
        {
            const uint8_t* krow0 = &k_lds[col * KROW + half * 32];
            const uint8_t* krow1 = krow0 + 32 * KROW;
            i32x8 fa[2], fb[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(krow0 + ks * 64);
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(krow0 + ks * 64 + 16);
                const u32x4 b0 = *reinterpret_cast<const u32x4*>(krow1 + ks * 64);
                const u32x4 b1 = *reinterpret_cast<const u32x4*>(krow1 + ks * 64 + 16);
                fa[ks] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                fb[ks] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                s[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[ks], qf[ks], s[0], 0, 0, 0, 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[ks], qf[ks], s[1], 0, 0, 0, 0, 0, 0);
            }
        }

        const int key0 = t * BN;
        const bool need_mask = (key0 + BN > p.sk) || (CAUSAL && key0 + BN - 1 > wave_row0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = key0 + kb * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
                    if (key >= p.sk || (CAUSAL && key > my_row)) s[kb][j] = kNegInf;
                }
            }
        }
        float mt = __builtin_fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int j = 2; j < 16; j += 2) mt = max3(mt, s[0][j], s[0][j + 1]);
#pragma unroll
        for (int j = 0; j < 16; j += 2) mt = max3(mt, s[1][j], s[1][j + 1]);
        mt = fmaxf(mt, swap_halves(mt));
        mt = mt == kNegInf ? kNegInf : mt * c;   // tile max in scaled base-2 units

        const float m_new = fmaxf(m_run, mt);
        const bool grow = m_new > m_run && (m_run == kNegInf || m_new - m_run > kRescaleThreshold);
        if (__any(grow)) {
            const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
            m_run = m_new;
        }
        // p' = p * scale_v = exp2(s*c - m + log2 scale_v): the V block scale rides in the exponent
        const float bias = (m_run == kNegInf ? 0.f : -m_run) + log2_sv;

        bf16x8 pf[4];
        float l_tile = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s0 = s[ks >> 1][(ks & 1) * 8 + 2 * i];
                const float s1 = s[ks >> 1][(ks & 1) * 8 + 2 * i + 1];
                float p0 = fast_exp2(fmaf(s0, c, bias));
                float p1 = fast_exp2(fmaf(s1, c, bias));
                if (need_mask) {
                    p0 = s0 == kNegInf ? 0.f : p0;
                    p1 = s1 == kNegInf ? 0.f : p1;
                }
                w[i] = pack_bf16x2(p0, p1);
                l_tile = add_bf16_pair(w[i], l_tile);
            }
            pf[ks] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
        l_run = fmaf(l_tile, inv_sv, l_run);   // back to unscaled probabilities

        {
            const uint16_t* vrow = &v_lds[col * VROW + half * 4];
            auto vfrag = [&](int cb, int ks) __attribute__((always_inline)) {
                const uint16_t* vr = vrow + cb * 32 * VROW + ks * 16;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
                return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            };
            bf16x8 a[2][CBLK];
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) a[0][cb] = vfrag(cb, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks + 1 < 4) {
#pragma unroll
                    for (int cb = 0; cb < CBLK; ++cb) a[(ks + 1) & 1][cb] = vfrag(cb, ks + 1);
                }
#pragma unroll
                for (int cb = 0; cb < CBLK; ++cb)
                    oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 1][cb], pf[ks], oacc[cb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    load_tile(0, std::integral_constant<int, 0>{});
    load_tile(1, std::integral_constant<int, 1>{});
    for (int t0 = 0; t0 < ntiles; t0 += PF) {
        auto step = [&](auto slot_c) __attribute__((always_inline)) {
            constexpr int slot = decltype(slot_c)::value;
            const int t = t0 + slot;
            if (t < ntiles) {
                __syncthreads();
                store_tile(slot_c);
                __syncthreads();
                load_tile(t + PF, slot_c);
                compute_tile(t);
            }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
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
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;   // m_run is already scaled
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
