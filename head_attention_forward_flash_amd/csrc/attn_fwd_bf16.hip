// Fused attention forward, bf16 in / bf16 out, fp32 accumulation, for gfx950.
//
// Computes O = softmax(scale * Q K^T + causal mask) V and the natural-log LSE per
// row: the MHA forward pass tuned on "Tune MHA config & small-head pipeline
// pathology" (Motivation; Technical Details: head-dim buckets 64, 128 and the
// dqk=192/dv=128 "pe" bucket; Profile 2: pipelining depth as the main lever).
//
// Work decomposition: one workgroup of 4 waves per (batch, query head, block of
// 128 query rows); each wave owns 32 query rows.  The kernel computes the
// TRANSPOSED scores S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that every lane
// holds one query row (lane % 32) and 32 of its keys per 64-key tile: the row
// max and row sum then stay in the lane except for one exchange with lane ^ 32,
// and the probabilities P^T are already laid out as the B operand of
// O^T = V^T P^T (the key order inside one 16-key MFMA step is permuted the same
// way on both operands, which leaves the contraction unchanged).
//
//   Q      32 rows x d_qk per wave, loaded once into registers (B operand).
//   K      64 x d_qk tile in LDS, row-major, rows padded by 16 bytes (A operand,
//          one ds_read_b128 per MFMA, conflict-free across 8 consecutive rows).
//   V      64 x d_v tile written TRANSPOSED into LDS (channel-major, keys
//          contiguous) so the A operand of O^T = V^T P^T is two ds_read_b64.
//   tiles  global -> registers for tile t+1 is issued before computing tile t
//          (register double buffering); LDS holds one tile.  Each tile's loads
//          use a buffer resource based at the tile, so their offsets are
//          loop-invariant and the hardware zero-fills keys past sk.
//   causal key tiles past the block's last row are never loaded; masking is
//          applied only on tiles that cross the diagonal or the ragged end.
//   softmax online, in base 2: p = exp2(s*c - m*c) with c = |scale| * log2 e
//          folded into one FMA (a negative scale negates Q, which is exact);
//          the running max is only moved when a row's max grows by more than
//          a factor 2^8 in probability, which keeps O and l consistent and
//          rescales rarely; the row sum adds the bf16-rounded probabilities
//          that enter P.V (v_dot2_f32_bf16), so O is normalised by exactly
//          the weights it was built from.
//
// Every global load goes through a buffer resource clamped to the (batch, head)
// slice, so rows past sq / sk read as zero instead of faulting.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mha {
namespace {

constexpr int BM = 128;       // query rows per workgroup
constexpr int BN = 64;        // keys per tile
constexpr int NTHREADS = 256;
constexpr float kRescaleThreshold = 8.0f;   // log2 units

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2) void attn_fwd_bf16_kernel(const AttnParams p) {
    // K/V tiles in flight: two for d_qk = 64 (short tiles cannot hide a load), else one
    constexpr int PF = DQK == 64 ? 2 : 1;
    constexpr int KROW = DQK + 8;             // K row in LDS, elements (16-byte pad)
    constexpr int VROW = BN + 4;              // V^T row in LDS, elements (8-byte pad)
    constexpr int KSTEPS = DQK / 16;          // MFMA k-steps for S^T
    constexpr int KCHUNKS = DQK / 32;         // 16-byte K chunks per thread per tile
    constexpr int VKEYS = DV / 32;            // keys per thread when staging V (4 or 2)
    constexpr int VKGROUPS = BN / VKEYS;      // key groups per tile
    constexpr int CBLK = DV / 32;             // 32-channel output blocks
    static_assert(BN * DQK / 8 == KCHUNKS * NTHREADS, "K staging must cover the tile");
    static_assert(VKGROUPS * (DV / 8) == NTHREADS, "V staging must cover the tile");

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[DV * VROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;     // query column of this lane in S^T / O^T
    const int half = lane >> 5;    // which half of the wave

    // ---- workgroup -> (batch, head, query block); consecutive logical ids stay on one XCD
    const int nwg = gridDim.x;
    const int nwg8 = nwg & ~7;
    const int pid = blockIdx.x;
    const int lid = pid < nwg8 ? (pid & 7) * (nwg8 >> 3) + (pid >> 3) : pid;
    const int mrev = lid % p.n_mblocks;
    const int bh = lid / p.n_mblocks;
    const int mblk = CAUSAL ? (p.n_mblocks - 1 - mrev) : mrev;   // causal: heavy blocks first
    const int h = bh % p.hq;
    const int bb = bh / p.hq;
    const int g = h / p.group;

    const char* qbase = static_cast<const char*>(p.q) + 2 * (bb * p.qv.sb + h * p.qv.sh);
    const char* kbase = static_cast<const char*>(p.k) + 2 * (bb * p.kv.sb + g * p.kv.sh);
    const char* vbase = static_cast<const char*>(p.v) + 2 * (bb * p.vv.sb + g * p.vv.sh);
    const auto qrs = make_rsrc(qbase, p.qv.slice_bytes);

    const int wave_row0 = mblk * BM + wave * 32;
    const int my_row = wave_row0 + col;

    // ---- Q fragment (B operand of S^T = K Q^T): lane holds Q[my_row][kk*16 + half*8 .. +8]
    bf16x8 qf[KSTEPS];
    {
        const uint32_t rowoff = my_row < p.sq ? static_cast<uint32_t>(my_row * p.qv.ss * 2) : kOutOfRange;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const uint32_t off = rowoff == kOutOfRange ? kOutOfRange : rowoff + (kk * 16 + half * 8) * 2;
            u32x4 w = buffer_load_b128(qrs, off);
            // softmax(c * s) with c < 0 equals softmax(|c| * (-s)): negate Q (exact) and use |c|
            if (p.scale_log2 < 0.f) w ^= 0x80008000u;
            qf[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }
    const float c = fabsf(p.scale_log2);   // base-2 score scale, >= 0

    const int kv_end = CAUSAL ? min(p.sk, (mblk + 1) * BM) : p.sk;
    const int ntiles = (kv_end + BN - 1) / BN;

    // ---- staging registers: PF tiles of K/V in flight (loads of tile t+PF are issued while
    //      tile t is computed)
    u32x4 kreg[PF][KCHUNKS];
    u32x4 vreg[PF][VKEYS];
    const int vkg = tid % VKGROUPS;   // key group (VKEYS consecutive keys)
    const int vcg = tid / VKGROUPS;   // 8-channel group

    // Per-thread byte offsets inside a tile (constant over the loop).  Each tile gets its own
    // buffer resource starting at its first key and clamped to the slice end, so keys past sk
    // (rows are disjoint: stride.s >= d, checked on the host) read as zero with no per-key test.
    uint32_t koff[KCHUNKS];
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
        const int chunk = tid + NTHREADS * i;
        koff[i] = static_cast<uint32_t>((chunk / (DQK / 8)) * p.kv.ss * 2 + (chunk % (DQK / 8)) * 16);
    }
    uint32_t voff[VKEYS];
#pragma unroll
    for (int i = 0; i < VKEYS; ++i) voff[i] = static_cast<uint32_t>((vkg * VKEYS + i) * p.vv.ss * 2 + vcg * 16);

    auto tile_rsrc = [&](const char* base, const View& vw, int t) __attribute__((always_inline)) {
        const int64_t start = static_cast<int64_t>(t) * BN * vw.ss * 2;
        const uint32_t left = start < static_cast<int64_t>(vw.slice_bytes)
                                  ? static_cast<uint32_t>(vw.slice_bytes - start) : 0u;
        return make_rsrc(left ? base + start : base, left);
    };
    auto load_tile = [&](int t, auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
        const auto kr = tile_rsrc(kbase, p.kv, t);
        const auto vr = tile_rsrc(vbase, p.vv, t);
#pragma unroll
        for (int i = 0; i < KCHUNKS; ++i) kreg[slot][i] = buffer_load_b128(kr, koff[i]);
#pragma unroll
        for (int i = 0; i < VKEYS; ++i) vreg[slot][i] = buffer_load_b128(vr, voff[i]);
    };
    auto store_tile = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int i = 0; i < KCHUNKS; ++i) {
            const int chunk = tid + NTHREADS * i;
            *reinterpret_cast<u32x4*>(&k_lds[(chunk / (DQK / 8)) * KROW + (chunk % (DQK / 8)) * 8]) = kreg[slot][i];
        }
        // V^T: channel (vcg*8 + e) row receives keys vkg*VKEYS .. +VKEYS
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int dw = e >> 1;
            const bool hi = e & 1;
            uint32_t w[VKEYS / 2];
#pragma unroll
            for (int i = 0; i < VKEYS / 2; ++i) {
                const uint32_t a = vreg[slot][2 * i][dw];
                const uint32_t c2 = vreg[slot][2 * i + 1][dw];
                w[i] = hi ? ((a >> 16) | (c2 & 0xffff0000u)) : ((a & 0xffffu) | (c2 << 16));
            }
            uint16_t* dst = &v_lds[(vcg * 8 + e) * VROW + vkg * VKEYS];
            if constexpr (VKEYS == 4) {
                *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
            } else {
                *reinterpret_cast<uint32_t*>(dst) = w[0];
            }
        }
    };

    f32x16 oacc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
    float m_run = kNegInf;   // running max of raw scores, same in lane and lane^32
    float l_run = 0.f;       // this lane's partial row sum over its half of the keys

    auto compute_tile = [&](int t) __attribute__((always_inline)) {
        // ---- S^T = K Q^T: two independent 32-key accumulators.  K fragments are read
        //      KAHEAD k-steps ahead of the MFMAs that use them; the scheduling fences keep
        //      the compiler from sinking the reads next to their use.
        f32x16 s[2] = {f32x16{}, f32x16{}};
        {
            constexpr int KAHEAD = 3;
            const uint16_t* krow0 = &k_lds[col * KROW + half * 8];
            const uint16_t* krow1 = krow0 + 32 * KROW;
            bf16x8 fa[KSTEPS], fb[KSTEPS];
#pragma unroll
            for (int kk = 0; kk < KAHEAD && kk < KSTEPS; ++kk) {
                fa[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow0 + kk * 16));
                fb[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow1 + kk * 16));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                if (kk + KAHEAD < KSTEPS) {
                    fa[kk + KAHEAD] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow0 + (kk + KAHEAD) * 16));
                    fb[kk + KAHEAD] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow1 + (kk + KAHEAD) * 16));
                }
                s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk], qf[kk], s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk], qf[kk], s[1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- mask (tiles crossing the diagonal or the ragged end only), tile max of raw scores
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

        // ---- online softmax with lazy rescaling (the reference max only moves when a row's
        //      max grows by more than 2^8 in probability)
        const float m_new = fmaxf(m_run, mt);
        const bool grow = m_new > m_run && (m_run == kNegInf || (m_new - m_run) * c > kRescaleThreshold);
        if (__any(grow)) {
            const float alpha = m_run == kNegInf ? 0.f : fast_exp2((m_run - m_new) * c);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
            m_run = m_new;
        }
        const float mc = (m_run == kNegInf) ? 0.f : m_run * c;

        bf16x8 pf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s0 = s[ks >> 1][(ks & 1) * 8 + 2 * i];
                const float s1 = s[ks >> 1][(ks & 1) * 8 + 2 * i + 1];
                float p0 = fast_exp2(fmaf(s0, c, -mc));
                float p1 = fast_exp2(fmaf(s1, c, -mc));
                if (need_mask) {   // masked keys give exactly 0 whatever c is
                    p0 = s0 == kNegInf ? 0.f : p0;
                    p1 = s1 == kNegInf ? 0.f : p1;
                }
                w[i] = pack_bf16x2(p0, p1);
                l_run = add_bf16_pair(w[i], l_run);   // the row sum of the rounded P fed to P.V
            }
            pf[ks] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }

        // ---- O^T += V^T P^T: per 16-key step, CBLK independent accumulators; the V
        //      fragments of step ks+1 are read while the MFMAs of step ks run
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

    // tiles past the last one load nothing (their buffer range is empty)
    load_tile(0, std::integral_constant<int, 0>{});
    if constexpr (PF > 1) load_tile(1, std::integral_constant<int, 1>{});
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
        if constexpr (PF > 1) step(std::integral_constant<int, 1>{});
    }

    // ---- epilogue: normalise, store O (bf16) and LSE
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
            const float lse = l_tot > 0.f ? (m_run * c + __log2f(l_tot)) * kLn2 : kNegInf;
            p.lse[(static_cast<int64_t>(bb) * p.hq + h) * p.sq + my_row] = lse;
        }
    }
}

template <int DQK, int DV, bool CAUSAL>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
    const int64_t nwg = static_cast<int64_t>(p.b) * p.hq * p.n_mblocks;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, CAUSAL>), dim3(static_cast<unsigned>(nwg)),
                       dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int attn_fwd_bf16_block_m() { return BM; }

hipError_t launch_attn_fwd_bf16(const AttnParams& p, int d_qk, int d_v, bool causal, hipStream_t stream) {
    if (d_qk == 64 && d_v == 64) return causal ? launch<64, 64, true>(p, stream) : launch<64, 64, false>(p, stream);
    if (d_qk == 128 && d_v == 128)
        return causal ? launch<128, 128, true>(p, stream) : launch<128, 128, false>(p, stream);
    if (d_qk == 192 && d_v == 128)
        return causal ? launch<192, 128, true>(p, stream) : launch<192, 128, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace mha
