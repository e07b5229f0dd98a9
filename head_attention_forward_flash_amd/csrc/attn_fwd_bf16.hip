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

constexpr float kRescaleThreshold = 8.0f;   // log2 units

// Tile shape per head-dim pair: BM query rows per workgroup (32 per wave), BN keys per tile,
// NSTAGE tiles in the LDS ring (NSTAGE - 1 in flight while one is computed).  128-row
// workgroups run two per CU (80 KiB of LDS each); the 256-row one runs alone with 8 waves.
// Chosen by A/B timing on MI355X: 256 rows halve the K/V traffic per FLOP, which pays off
// for the wide d192/d128 tiles; three stages help only the short d64 tiles.
template <int DQK, int DV> struct TileCfg;
template <> struct TileCfg<64, 64> { static constexpr int BM = 128, BN = 64, NSTAGE = 3; };
template <> struct TileCfg<128, 128> { static constexpr int BM = 128, BN = 64, NSTAGE = 2; };
template <> struct TileCfg<192, 128> { static constexpr int BM = 256, BN = 64, NSTAGE = 2; };

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__((TileCfg<DQK, DV>::BM * 2), 2) void attn_fwd_bf16_kernel(const AttnParams p) {
    constexpr int BM = TileCfg<DQK, DV>::BM;           // query rows per workgroup
    constexpr int NTHREADS = BM * 2;                   // one wave per 32 rows
    constexpr int NWAVES = NTHREADS / 64;
    constexpr int BN = TileCfg<DQK, DV>::BN;           // keys per tile
    constexpr int NSTAGE = TileCfg<DQK, DV>::NSTAGE;
    constexpr int KB = BN / 32;                        // 32-key blocks per tile
    constexpr int KROWB = DQK * 2;            // bytes per K row in LDS (16-byte chunks XOR-swizzled)
    constexpr int VROWB = DV * 2;             // bytes per V row in LDS (row-major, swizzled)
    constexpr int KTILE = BN * KROWB;
    constexpr int VTILE = BN * VROWB;
    constexpr int STAGE = KTILE + VTILE;      // one LDS stage: a K tile then a V tile
    constexpr int KDMA = KTILE / 1024 / NWAVES;   // 1 KiB DMA blocks per wave per K tile
    constexpr int VDMA = VTILE / 1024 / NWAVES;
    constexpr int KSTEPS = DQK / 16;          // MFMA k-steps for S^T
    constexpr int CBLK = DV / 32;             // 32-channel output blocks
    static_assert(KDMA * NWAVES * 1024 == KTILE && VDMA * NWAVES * 1024 == VTILE, "DMA blocks must cover the tiles");

    static_assert(NSTAGE >= 2 && NSTAGE <= 4, "ring of 2 to 4 stages");
    static_assert(NSTAGE * STAGE <= (BM == 128 ? 80 : 160) * 1024, "the workgroups of a CU must fit in LDS");
    // The stages are distinct LDS objects: the compiler's wait insertion then knows that the
    // DMA filling one stage cannot alias the fragment reads of another, and does not make the
    // computation of tile t wait for the loads of later tiles.
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[NSTAGE > 2 ? STAGE : 1024];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[NSTAGE > 3 ? STAGE : 1024];
    auto stage_ptr = [&](auto i_c) __attribute__((always_inline)) -> uint8_t* {
        constexpr int i = decltype(i_c)::value % NSTAGE;
        if constexpr (i == 0) return lds0;
        else if constexpr (i == 1) return lds1;
        else if constexpr (i == 2) return lds2;
        else return lds3;
    };

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

    // ---- K/V tiles go global -> LDS by DMA (buffer_load ... lds): lane l of a wave writes
    //      16 bytes at block base + 16*l, and its global address decides what lands there.
    //      Rows are unpadded and their 16-byte chunks XOR-swizzled so that the fragment reads
    //      below are bank-conflict free on gfx950's LDS, which serves 256 bytes per clock
    //      (16 lanes of a b128 read, 32 lanes of a b64 read):
    //        K: the 16 rows one b128 read touches land on 16 distinct 16-byte bank groups;
    //        V: the 4 rows one transposing read touches land on 4 distinct 64-byte quarters.
    //      The per-lane global offsets are loop-invariant; each tile's buffer descriptor is
    //      based at the tile and bounded by the slice, so keys past sk land as zeros.
    auto kswz = [](int r) __attribute__((always_inline)) {
        return KROWB % 256 == 0 ? (r & 15) : ((r >> 1) & 7);    // rows of 256 B, else 128/384 B
    };
    auto vswz = [](int r) __attribute__((always_inline)) {
        return VROWB % 256 == 0 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
    };
    uint32_t kgo[KDMA], vgo[VDMA];
#pragma unroll
    for (int i = 0; i < KDMA; ++i) {
        const int pos = (wave * KDMA + i) * 1024 + lane * 16;
        const int r = pos / KROWB, pc = (pos % KROWB) / 16;
        kgo[i] = static_cast<uint32_t>(r * p.kv.ss * 2 + ((pc ^ kswz(r)) * 16));
    }
#pragma unroll
    for (int i = 0; i < VDMA; ++i) {
        const int pos = (wave * VDMA + i) * 1024 + lane * 16;
        const int r = pos / VROWB, pc = (pos % VROWB) / 16;
        vgo[i] = static_cast<uint32_t>(r * p.vv.ss * 2 + ((pc ^ vswz(r)) * 16));
    }
    auto tile_rsrc = [&](const char* base, const View& vw, int t) __attribute__((always_inline)) {
        const int64_t start = static_cast<int64_t>(t) * BN * vw.ss * 2;
        const uint32_t left = start < static_cast<int64_t>(vw.slice_bytes)
                                  ? static_cast<uint32_t>(vw.slice_bytes - start) : 0u;
        return make_rsrc(left ? base + start : base, left);
    };
    auto issue_tile = [&](int t, uint8_t* stage_base) __attribute__((always_inline)) {
        const auto kr = tile_rsrc(kbase, p.kv, t);
        const auto vr = tile_rsrc(vbase, p.vv, t);
        uint8_t* kd = stage_base + wave * KDMA * 1024;
        uint8_t* vd = stage_base + KTILE + wave * VDMA * 1024;
#pragma unroll
        for (int i = 0; i < KDMA; ++i)
            buffer_load_lds_b128(kr, kd + i * 1024, kgo[i]);
#pragma unroll
        for (int i = 0; i < VDMA; ++i)
            buffer_load_lds_b128(vr, vd + i * 1024, vgo[i]);
    };

    // LDS starts as zeros so that any row the DMA does not fill holds finite values
    for (int i = tid; i < STAGE / 16; i += NTHREADS) {
        reinterpret_cast<u32x4*>(lds0)[i] = u32x4{0, 0, 0, 0};
        reinterpret_cast<u32x4*>(lds1)[i] = u32x4{0, 0, 0, 0};
        if constexpr (NSTAGE > 2) reinterpret_cast<u32x4*>(lds2)[i] = u32x4{0, 0, 0, 0};
        if constexpr (NSTAGE > 3) reinterpret_cast<u32x4*>(lds3)[i] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();

    f32x16 oacc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
    float m_run = kNegInf;   // running max of raw scores, same in lane and lane^32
    float l_run = 0.f;       // this lane's partial row sum over its half of the keys

    // fragment addresses inside a stage (bytes)
    const int kx = kswz(col);                     // the row's chunk swizzle (same for every block)
    const int t16 = lane & 15;
    // V transposing reads: lane t of a 16-lane group points at key (k0 + t/4), channel
    // (c0 + 4*(t%4)); the group then receives, lane by lane, 16 consecutive channels of 4 keys.
    const int vkey_l = half * 4 + (t16 >> 2);                 // key offset inside a 16-key step
    const int vch_l = ((lane >> 4) & 1) * 16 + 4 * (t16 & 3); // channel offset inside a 32-block

    auto compute_tile = [&](int t, const uint8_t* kl) __attribute__((always_inline)) {
        const uint8_t* vl = kl + KTILE;

        // ---- S^T = K Q^T: KB independent 32-key accumulators; K fragments are read KAHEAD
        //      k-steps ahead of the MFMAs that use them
        f32x16 s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
        {
            constexpr int KAHEAD = 3;
            auto kfrag = [&](int kb, int kk) __attribute__((always_inline)) {
                const int chunk = (kk * 2 + half) ^ kx;
                return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kl + (kb * 32 + col) * KROWB + chunk * 16));
            };
            bf16x8 fr[KSTEPS][KB];
#pragma unroll
            for (int kk = 0; kk < KAHEAD && kk < KSTEPS; ++kk)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) fr[kk][kb] = kfrag(kb, kk);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                if (kk + KAHEAD < KSTEPS) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) fr[kk + KAHEAD][kb] = kfrag(kb, kk + KAHEAD);
                }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[kk][kb], qf[kk], s[kb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- mask (tiles crossing the diagonal or the ragged end only), tile max of raw scores
        const int key0 = t * BN;
        const bool need_mask = (key0 + BN > p.sk) || (CAUSAL && key0 + BN - 1 > wave_row0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
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
        for (int kb = 1; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; j += 2) mt = max3(mt, s[kb][j], s[kb][j + 1]);
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

        constexpr int PSTEPS = BN / 16;   // 16-key MFMA steps of P.V
        bf16x8 pf[PSTEPS];
#pragma unroll
        for (int ks = 0; ks < PSTEPS; ++ks) {
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

        // ---- O^T += V^T P^T: the A operand (32 channels x 16 keys) comes from two transposing
        //      reads of row-major V; keys ks*16 + {half*4 .. +3} and {8 + half*4 .. +3} match
        //      the key order of P^T's B operand.  Fragments of step ks+1 are read during step ks.
        {
            auto vfrag = [&](int cb, int ks) __attribute__((always_inline)) {
                u32x2 part[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int key = ks * 16 + r * 8 + vkey_l;
                    const int ch = cb * 32 + vch_l;
                    const int chunk = (ch >> 3) ^ vswz(key);
                    const uint8_t* a = vl + key * VROWB + chunk * 16 + (ch & 7) * 2;
                    part[r] = lds_read_tr16_b64(a);
                }
                return __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
            };
            bf16x8 a[2][CBLK];
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) a[0][cb] = vfrag(cb, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < PSTEPS; ++ks) {
                if (ks + 1 < PSTEPS) {
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

    // ---- main loop: NSTAGE - 1 tiles stream into the ring while tile t is computed.  The
    //      barrier makes every wave's part of tile t visible and guarantees that every wave
    //      finished tile t - 1, whose stage the next DMA overwrites.
    constexpr int DMA_PER_TILE = KDMA + VDMA;
    constexpr int VM_LEFT = (NSTAGE - 2) * DMA_PER_TILE;   // DMAs of younger tiles still in flight
    static_assert(VM_LEFT < 64, "vmcnt is 6 bits");
    constexpr int WAIT_TILE = (VM_LEFT & 15) | ((VM_LEFT >> 4) << 14) | 0x0F70;   // vmcnt(VM_LEFT)
    auto prologue = [&](auto i_c) __attribute__((always_inline)) {
        if constexpr (decltype(i_c)::value < NSTAGE - 1) issue_tile(decltype(i_c)::value, stage_ptr(i_c));
    };
    prologue(std::integral_constant<int, 0>{});
    prologue(std::integral_constant<int, 1>{});
    prologue(std::integral_constant<int, 2>{});
    for (int t0 = 0; t0 < ntiles; t0 += NSTAGE) {
        auto step = [&](auto j_c) __attribute__((always_inline)) {
            constexpr int j = decltype(j_c)::value;
            const int t = t0 + j;
            if (j < NSTAGE && t < ntiles) {
                __builtin_amdgcn_s_waitcnt(WAIT_TILE);   // this wave's part of tile t has landed
                __syncthreads();
                // past the last tile: empty buffer range, nothing is read
                issue_tile(t + NSTAGE - 1, stage_ptr(std::integral_constant<int, j + NSTAGE - 1>{}));
                compute_tile(t, stage_ptr(j_c));
            }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        if constexpr (NSTAGE > 2) step(std::integral_constant<int, 2>{});
        if constexpr (NSTAGE > 3) step(std::integral_constant<int, 3>{});
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
hipError_t launch(AttnParams p, hipStream_t stream) {
    constexpr int BM = TileCfg<DQK, DV>::BM;
    p.n_mblocks = (p.sq + BM - 1) / BM;
    const int64_t nwg = static_cast<int64_t>(p.b) * p.hq * p.n_mblocks;
    if (nwg == 0) return hipSuccess;
    if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, CAUSAL>), dim3(static_cast<unsigned>(nwg)),
                       dim3(BM * 2), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnParams& p, int d_qk, int d_v, bool causal, hipStream_t stream) {
    if (d_qk == 64 && d_v == 64) return causal ? launch<64, 64, true>(p, stream) : launch<64, 64, false>(p, stream);
    if (d_qk == 128 && d_v == 128)
        return causal ? launch<128, 128, true>(p, stream) : launch<128, 128, false>(p, stream);
    if (d_qk == 192 && d_v == 128)
        return causal ? launch<192, 128, true>(p, stream) : launch<192, 128, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace mha
