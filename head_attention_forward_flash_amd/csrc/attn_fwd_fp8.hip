// Attention forward on E4M3-quantised, K-smoothed inputs (d = 128), gfx950.
//
// The attention side of the FP8 hd128 mha_v4 recipe ("[HIP] Mha v4: run the
// K-smoothing gate as one HIP call", Performance table; "MHA v4: fixes,
// refactor, new kernel, perf tweaks", BF16/FP8 recipe).  Inputs are written by
// quant_fp8: E4M3 codes of Q and K - mean, the E4M3 values of V widened exactly
// to bf16, and one fp32 scale per (batch, head, 128-token block) for each.
//
// Same pipeline as the bf16 kernel (4 waves x 32 query rows, 64-key tiles, one
// query per lane in S^T, K/V tiles staged into a ring of LDS stages by DMA):
//   S^T = K8 Q8^T  on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulate),
//                  two k-steps of 64 channels; both operands read 32 bytes of
//                  their row per lane, so the MFMA's channel order cancels out;
//   scores         t = s * (scale_q * scale_k * |softmax_scale| * log2 e): one
//                  factor per tile, since a 64-key tile sits inside one
//                  128-token scale block and the 128 query rows are one block;
//                  the factor and the running max fold into one FMA before exp2;
//   P.V            on bf16 MFMA; the V operand comes from transposing LDS reads of
//                  the widened V values, and the V block scale enters P through
//                  the exponent (p' = exp2(t - m + log2 scale_v)) before P is
//                  rounded to bf16;
//   l              sums the bf16 P' fed to P.V (v_dot2_f32_bf16), divided by the
//                  tile's V scale once per tile.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mha {
namespace {

constexpr int BM = 128;          // query rows per workgroup = one Q scale block
constexpr int BN = 64;           // keys per tile (half a K/V scale block)
constexpr int D = 128;
constexpr int NTHREADS = 256;
constexpr int NSTAGE = 3;
constexpr float kRescaleThreshold = 8.0f;

template <bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2) void attn_fwd_fp8_kernel(const Fp8AttnParams p) {
    constexpr int KROWB = D;                  // bytes per K8 row
    constexpr int VROWB = D * 2;              // bytes per widened V row
    constexpr int KTILE = BN * KROWB;
    constexpr int VTILE = BN * VROWB;
    constexpr int STAGE = KTILE + VTILE;
    constexpr int KDMA = KTILE / 1024 / 4;    // 1 KiB DMA blocks per wave per tile
    constexpr int VDMA = VTILE / 1024 / 4;
    constexpr int CBLK = D / 32;
    static_assert(KDMA * 4 * 1024 == KTILE && VDMA * 4 * 1024 == VTILE, "DMA blocks must cover the tiles");
    static_assert(NSTAGE * STAGE <= 80 * 1024, "two workgroups per CU must fit in LDS");

    // distinct LDS objects per stage (see the bf16 kernel: keeps the DMA of later tiles from
    // gating the fragment reads of the current one)
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[STAGE];
    auto stage_ptr = [&](auto i_c) __attribute__((always_inline)) -> uint8_t* {
        constexpr int i = decltype(i_c)::value % NSTAGE;
        if constexpr (i == 0) return lds0;
        else if constexpr (i == 1) return lds1;
        else return lds2;
    };

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
    const uint32_t kslice = static_cast<uint32_t>(p.nk) * BM * KROWB;
    const uint32_t vslice = static_cast<uint32_t>(p.nk) * BM * VROWB;
    const auto qrs = make_rsrc(p.q + static_cast<int64_t>(bh) * qslice, qslice);
    const uint8_t* kbase = p.k + static_cast<int64_t>(bg) * kslice;
    const uint8_t* vbase = p.v + static_cast<int64_t>(bg) * vslice;
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

    // ---- DMA layout (see the bf16 kernel): K8 rows of 128 B keep chunk c of row r at
    //      c ^ ((r >> 1) & 7); widened V rows of 256 B keep chunk c of key r at c ^ 4*(r & 3).
    auto kswz = [](int r) __attribute__((always_inline)) { return (r >> 1) & 7; };
    auto vswz = [](int r) __attribute__((always_inline)) { return (r & 3) << 2; };
    uint32_t kgo[KDMA], vgo[VDMA];
#pragma unroll
    for (int i = 0; i < KDMA; ++i) {
        const int pos = (wave * KDMA + i) * 1024 + lane * 16;
        const int r = pos / KROWB, pc = (pos % KROWB) / 16;
        kgo[i] = static_cast<uint32_t>(r * KROWB + (pc ^ kswz(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < VDMA; ++i) {
        const int pos = (wave * VDMA + i) * 1024 + lane * 16;
        const int r = pos / VROWB, pc = (pos % VROWB) / 16;
        vgo[i] = static_cast<uint32_t>(r * VROWB + (pc ^ vswz(r)) * 16);
    }
    auto tile_rsrc = [&](const uint8_t* base, uint32_t slice, uint32_t rowb, int t) __attribute__((always_inline)) {
        const uint32_t start = static_cast<uint32_t>(t) * BN * rowb;
        const uint32_t left = start < slice ? slice - start : 0u;
        return make_rsrc(left ? base + start : base, left);
    };
    auto issue_tile = [&](int t, uint8_t* stage_base) __attribute__((always_inline)) {
        // tiles past the padded key range read nothing (empty buffer range)
        const auto kr = tile_rsrc(kbase, kslice, KROWB, t);
        const auto vr = tile_rsrc(vbase, vslice, VROWB, t);
        uint8_t* kd = stage_base + wave * KDMA * 1024;
        uint8_t* vd = stage_base + KTILE + wave * VDMA * 1024;
#pragma unroll
        for (int i = 0; i < KDMA; ++i) buffer_load_lds_b128(kr, kd + i * 1024, kgo[i]);
#pragma unroll
        for (int i = 0; i < VDMA; ++i) buffer_load_lds_b128(vr, vd + i * 1024, vgo[i]);
    };

    for (int i = tid; i < STAGE / 16; i += NTHREADS) {
        reinterpret_cast<u32x4*>(lds0)[i] = u32x4{0, 0, 0, 0};
        reinterpret_cast<u32x4*>(lds1)[i] = u32x4{0, 0, 0, 0};
        reinterpret_cast<u32x4*>(lds2)[i] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();

    f32x16 oacc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
    float m_run = kNegInf;   // running max in base-2 units of scaled scores
    float l_run = 0.f;

    const int kx = kswz(col);
    const int t16 = lane & 15;
    const int vkey_l = half * 4 + (t16 >> 2);
    const int vch_l = ((lane >> 4) & 1) * 16 + 4 * (t16 & 3);

    auto compute_tile = [&](int t, const uint8_t* kl) __attribute__((always_inline)) {
        const uint8_t* vl = kl + KTILE;
        const int kblk = (t * BN) / BM;
        const float c = cq * k_scale[kblk];            // this tile's base-2 score factor
        const float log2_sv = __log2f(v_scale[kblk]);  // V block scale, folded into P
        const float inv_sv = 1.f / v_scale[kblk];

        // ---- S^T = K8 Q8^T: two 32-key accumulators, two k-steps of 64 channels
        f32x16 s[2] = {f32x16{}, f32x16{}};
        {
            i32x8 fr[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint8_t* row = kl + (kb * 32 + col) * KROWB;
                    const int c0 = (ks * 4 + half * 2) ^ kx, c1 = (ks * 4 + half * 2 + 1) ^ kx;
                    const u32x4 a0 = *reinterpret_cast<const u32x4*>(row + c0 * 16);
                    const u32x4 a1 = *reinterpret_cast<const u32x4*>(row + c1 * 16);
                    fr[ks][kb] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                       (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[ks][kb], qf[ks], s[kb], 0, 0, 0, 0, 0, 0);
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

        // ---- O^T += V^T P'^T from transposing reads of the widened V rows
        {
            auto vfrag = [&](int cb, int ks) __attribute__((always_inline)) {
                u32x2 part[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int key = ks * 16 + r * 8 + vkey_l;
                    const int ch = cb * 32 + vch_l;
                    const int chunk = (ch >> 3) ^ vswz(key);
                    part[r] = lds_read_tr16_b64(vl + key * VROWB + chunk * 16 + (ch & 7) * 2);
                }
                return __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
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

    // ---- main loop: NSTAGE - 1 tiles stream into the ring while tile t is computed
    constexpr int VM_LEFT = (NSTAGE - 2) * (KDMA + VDMA);
    static_assert(VM_LEFT < 16, "vmcnt immediate");
    constexpr int WAIT_TILE = VM_LEFT | 0x0F70;
    issue_tile(0, lds0);
    issue_tile(1, lds1);
    for (int t0 = 0; t0 < ntiles; t0 += NSTAGE) {
        auto step = [&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            const int t = t0 + j;
            if (t < ntiles) {
                __builtin_amdgcn_s_waitcnt(WAIT_TILE);   // this wave's part of tile t has landed
                __syncthreads();
                issue_tile(t + NSTAGE - 1, stage_ptr(std::integral_constant<int, j + NSTAGE - 1>{}));
                compute_tile(t, stage_ptr(j_c));
            }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
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
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;   // m_run is scaled
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
