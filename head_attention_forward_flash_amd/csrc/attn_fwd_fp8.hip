// Attention forward on E4M3-quantised, K-smoothed inputs (d = 64 or 128), gfx950.
//
// The attention side of the FP8 hd128 mha_v4 recipe ("[HIP] Mha v4: run the
// K-smoothing gate as one HIP call", Performance table; "MHA v4: fixes,
// refactor, new kernel, perf tweaks", BF16/FP8 recipe).  Inputs are written by
// quant_fp8: E4M3 codes of Q and K - mean, the E4M3 values of V widened exactly
// to bf16, and one fp32 scale per (batch, head, 128-token block) for each.
//
// Same organisation as the bf16 kernel (4 waves x 32 query rows, 64-key tiles,
// one query per lane in S^T, K and V tiles streamed by DMA into two-slot LDS
// rings, the loop software-pipelined over 32-key blocks):
//   S^T = K8 Q8^T  on v_mfma_scale_f32_32x32x64_f8f6f4 with zero scales (plain
//                  E4M3 x E4M3, fp32 accumulate), two k-steps of 64 channels;
//                  both operands read 32 bytes of their row per lane, so the
//                  MFMA's channel order cancels out;
//   scores         t = s * (scale_q * scale_k * |softmax_scale| * log2 e): one
//                  factor per tile, since a 64-key tile sits inside one
//                  128-token scale block and the 128 query rows are one block;
//                  the running max is kept in these scaled base-2 units;
//   P.V            on bf16 MFMA; the V operand comes from transposing LDS reads of
//                  the widened V values, and the V block scale enters P through
//                  the exponent (p' = exp2(t - m + log2 scale_v)) before P is
//                  rounded to bf16;
//   l              sums the bf16 P' fed to P.V (v_dot2_f32_bf16), divided by the
//                  V scale of its block.
// Masked scores are -inf; the per-tile factor is at least FLT_MIN, so they reach
// the exponential as -inf and come out as exactly 0.
//
// MXFP8 (MX = true): Q and K codes carry one E8M0 exponent per 32 channels of a
// row instead of block scales, which go in as the scaled MFMA's per-lane scale
// operands, so S comes out fully scaled.  The instruction applies the scale of
// lane r (r < 32) to the first 16 bytes of lanes r AND r + 32, and that of lane
// r + 32 to their last 16 bytes (measured), so in a 64-channel k-step lane half
// h holds channels [16h, 16h + 16) and [32 + 16h, 32 + 16h + 16): the first 32
// channels then get lane r's scale, the next 32 lane r + 32's.  V arrives with
// its exponents applied, so the per-tile factor is the softmax scale alone and
// P carries no V scale.

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "kernels.h"

namespace mha {
namespace {

// max(x of this lane, x of lane ^ 32): the exchange of max_with_partner followed by one v_max
// (x likewise must not come straight from an MFMA).
__device__ __forceinline__ float max_halves(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_max_f32 %0, %0, %1" : "+v"(a), "+v"(b));
    return a;
}

constexpr int BM = 128;          // query rows per workgroup = one Q scale block
constexpr int BN = 64;           // keys per tile (half a K/V scale block)
constexpr int NTHREADS = 256;
// A lane's sum of the 16 probabilities of a block it computed against the reference max: at most
// this, each probability is at most 2^8 (the reference lags the row max by at most 8 in log2
// units), otherwise the block takes a new reference.
constexpr float kSumLimit = 256.0f;
// Score pairs (of 8 per lane and block) of block u+1 whose exponentials run under the P.V MFMAs
// of block u (see the main loop).
#ifndef MHA_FP8_EARLY
#define MHA_FP8_EARLY 5
#endif
// Query blocks per workgroup on non-causal d128 grids (see RB below); 1 turns it off
#ifndef MHA_FP8_BLOCKS_PER_WG
#define MHA_FP8_BLOCKS_PER_WG 2
#endif
constexpr int EARLY = MHA_FP8_EARLY;
template <int N> using IC = std::integral_constant<int, N>;
constexpr float kMinFactor = 1.17549435e-38f;   // FLT_MIN

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kGrpValu = 0x002, kGrpMfma = 0x008, kGrpVmem = 0x010, kGrpDsRead = 0x100;

template <int I, int VMEM, int DS_SLOTS, int DS_PER, int VALU_SLOTS, int VALU_PER>
__device__ __forceinline__ void sched_slot() {
    __builtin_amdgcn_sched_group_barrier(kGrpMfma, 1, 0);
    if constexpr (I < VMEM) __builtin_amdgcn_sched_group_barrier(kGrpVmem, 1, 0);
    if constexpr (I < DS_SLOTS) __builtin_amdgcn_sched_group_barrier(kGrpDsRead, DS_PER, 0);
    if constexpr (I < VALU_SLOTS) __builtin_amdgcn_sched_group_barrier(kGrpValu, VALU_PER, 0);
}

// MFMAS matrix instructions, DS_PRE reads first, the other DS reads DS_PER per MFMA, VMEM
// instructions one per MFMA, VALU instructions spread evenly.
template <int MFMAS, int DS_TOTAL, int DS_PRE, int DS_PER, int VALU, int VMEM, int... I>
__device__ __forceinline__ void sched_region(std::integer_sequence<int, I...>) {
    constexpr int DS_SLOTS = (DS_TOTAL - DS_PRE) / DS_PER;
    constexpr int VALU_PER = (VALU + MFMAS - 1) / MFMAS;
    constexpr int VALU_SLOTS = VALU_PER > 0 ? (VALU + VALU_PER - 1) / VALU_PER : 0;
    if constexpr (DS_PRE > 0) __builtin_amdgcn_sched_group_barrier(kGrpDsRead, DS_PRE, 0);
    (sched_slot<I, VMEM, DS_SLOTS, DS_PER, VALU_SLOTS, VALU_PER>(), ...);
}

// RB: query blocks of one head per workgroup.  Non-causal grids that still fill the device give a
// workgroup of RB x 4 waves RB consecutive blocks, which share every K/V tile the DMA brings in
// (each wave's rows and registers stay as with one block).
template <int D, bool CAUSAL, bool MX, int RB = 1>
__global__ __launch_bounds__(NTHREADS * RB, D == 64 ? 3 : RB > 1 ? 1 : 2) void attn_fwd_fp8_kernel(const Fp8AttnParams p) {
    static_assert(RB == 1 || !CAUSAL, "causal grids pair blocks instead");
    constexpr int NWAVES = NTHREADS * RB / 64;
    constexpr int KROWB = D;                  // bytes per K8 row
    constexpr int VROWB = D * 2;              // bytes per widened V row
    constexpr int KTILE = BN * KROWB;
    constexpr int VTILE = BN * VROWB;
    constexpr int KDMA = KTILE / 1024 / NWAVES;   // 1 KiB DMA blocks per wave per tile
    constexpr int VDMA = VTILE / 1024 / NWAVES;
    constexpr int CBLK = D / 32;
    constexpr int KS = D / 64;                // fp8 MFMA k-steps of 64 channels
    constexpr int EB = D / 32;                // MXFP8 exponent bytes per row
    static_assert(KDMA * NWAVES * 1024 == KTILE && VDMA * NWAVES * 1024 == VTILE, "DMA blocks must cover the tiles");
    static_assert(2 * (KTILE + VTILE) <= 80 * 1024, "two workgroups per CU must fit in LDS");

    // each ring slot is its own LDS object, so a DMA into one slot never gates the fragment
    // reads of another in the compiler's wait insertion
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[KTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[VTILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[VTILE];
    auto k_slot = [&](auto i_c) __attribute__((always_inline)) -> uint8_t* {
        if constexpr (decltype(i_c)::value % 2 == 0) return k_lds0;
        else return k_lds1;
    };
    auto v_slot = [&](auto i_c) __attribute__((always_inline)) -> uint8_t* {
        if constexpr (decltype(i_c)::value % 2 == 0) return v_lds0;
        else return v_lds1;
    };

    // ---- workgroup -> (batch, head, query block); consecutive logical ids stay on one XCD.
    //      Causal grids pair the query blocks of a head (as the bf16 kernel does): a workgroup
    //      takes block n-1-j and then block j, so every workgroup does the same work.
    const int nwg = gridDim.x;
    const int nwg8 = nwg & ~7;
    const int pid = blockIdx.x;
    const int lid = pid < nwg8 ? (pid & 7) * (nwg8 >> 3) + (pid >> 3) : pid;
    const int per_head = CAUSAL ? (p.n_mblocks + 1) / 2 : (p.n_mblocks + RB - 1) / RB;
    const int mrev = lid % per_head;
    const int bh = lid / per_head;
    int mblk = CAUSAL ? (p.n_mblocks - 1 - mrev) : mrev * RB;   // causal: the heavy block first
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
    const float* k_scale = MX ? nullptr : p.k_scale + static_cast<int64_t>(bg) * p.nk;
    const float* v_scale = MX ? nullptr : p.v_scale + static_cast<int64_t>(bg) * p.nk;
    // MXFP8 exponents: 4 bytes per row (one per 32 channels), rows padded like the codes
    const uint32_t exp_slice = static_cast<uint32_t>(p.nk) * BM * EB;
    const auto kers = make_rsrc(MX ? p.k_exps + static_cast<int64_t>(bg) * exp_slice : nullptr, MX ? exp_slice : 0u);

    // LDS starts as zeros so that any row the DMA does not fill holds finite values
    for (int i = threadIdx.x; i < KTILE / 16; i += NTHREADS * RB) {
        reinterpret_cast<u32x4*>(k_lds0)[i] = u32x4{0, 0, 0, 0};
        reinterpret_cast<u32x4*>(k_lds1)[i] = u32x4{0, 0, 0, 0};
    }
    for (int i = threadIdx.x; i < VTILE / 16; i += NTHREADS * RB) {
        reinterpret_cast<u32x4*>(v_lds0)[i] = u32x4{0, 0, 0, 0};
        reinterpret_cast<u32x4*>(v_lds1)[i] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();

next_item:
    // A pair's second block passes the lane index through an empty asm statement: nothing derived
    // from it is then hoisted out of the loop over the pair, where it would stay live across every
    // tile and crowd the tile loop's registers.
    {
    int tid = threadIdx.x;
    if constexpr (CAUSAL) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;
    const int half = lane >> 5;

    // the wave's query block (RB > 1: the workgroup's blocks mblk, mblk + 1, ...; one past the
    // last block holds no rows: its Q reads as zeros and nothing of it is stored)
    const int wblk = RB == 1 ? mblk : mblk + wave / 4;
    const int wave_row0 = wblk * BM + (RB == 1 ? wave : wave % 4) * 32;
    const int my_row = wave_row0 + col;

    // Q8 fragment: two k-steps of 64 channels, 32 codes per lane each.  softmax(c*s) with
    // c < 0 equals softmax(|c| * (-s)): a negative scale flips the sign bits of Q (exact).
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80808080u : 0u;
    i32x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        // plain fp8: channels [32h, 32h + 32) of the k-step; MXFP8: [16h, +16) and [32 + 16h, +16)
        const uint32_t off = static_cast<uint32_t>(my_row * D + ks * 64 + half * (MX ? 16 : 32));
        const u32x4 a = buffer_load_b128(qrs, off) ^ qsign;
        const u32x4 b = buffer_load_b128(qrs, off + (MX ? 32 : 16)) ^ qsign;
        qf[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
    const float q_scale = MX || wblk >= p.nq ? 1.f : p.q_scale[static_cast<int64_t>(bh) * p.nq + wblk];
    const float cq = q_scale * fabsf(p.scale_log2);   // base-2 factor of this block's scores, >= 0
    // MXFP8: the E8M0 byte of each k-step's 32 channels of this lane's query, in bits 0-7
    uint32_t qe[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qe[ks] = 0u;
    // the row's EB exponent bytes (d128: 4, one dword; d64: 2)
    auto exp_word = [&](__amdgpu_buffer_rsrc_t r, uint32_t row) __attribute__((always_inline)) -> uint32_t {
        if constexpr (EB == 4) return buffer_load_b32(r, row * 4);
        else return buffer_load_b16(r, row * 2);
    };
    if constexpr (MX) {
        const uint32_t qslice_e = static_cast<uint32_t>(p.nq) * BM * EB;
        const auto qers = make_rsrc(p.q_exps + static_cast<int64_t>(bh) * qslice_e, qslice_e);
        const uint32_t w = exp_word(qers, static_cast<uint32_t>(my_row));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qe[ks] = w >> (8 * (2 * ks + half));
    }
    // MXFP8: the exponent words of this lane's key in the two 32-key blocks of tile t (zeros
    // past the padded key range)
    auto kexp_load = [&](int t) __attribute__((always_inline)) {
        const uint32_t key = static_cast<uint32_t>(t * BN + col);
        return u32x2{exp_word(kers, key), exp_word(kers, key + 32)};
    };

    const int kv_end = CAUSAL ? min(p.sk, (mblk + 1) * BM) : p.sk;
    const int ntiles = (kv_end + BN - 1) / BN;

    // per-tile factors: the scores' base-2 factor (>= FLT_MIN) and the V block scale
    struct TileScale {
        float c, log2_sv, inv_sv;
    };
    auto tile_scale = [&](int t) __attribute__((always_inline)) {
        if constexpr (MX) {
            return TileScale{fmaxf(cq, kMinFactor), 0.f, 1.f};
        } else {
            const int kblk = min((t * BN) / BM, p.nk - 1);   // past the last tile: any valid block
            const float sv = v_scale[kblk];
            // 1/sv only rescales the row sum: the hardware reciprocal (1 ulp) is enough
            return TileScale{fmaxf(cq * k_scale[kblk], kMinFactor), __log2f(sv), __builtin_amdgcn_rcpf(sv)};
        }
    };

    // ---- DMA layout (see the bf16 kernel): K8 rows of 128 B keep chunk c of row r at
    //      c ^ ((r >> 1) & 7); widened V rows of 256 B keep chunk c of key r at c ^ 4*(r & 3).
    // (d64: K8 rows of 64 B keep chunk c at c ^ ((r >> 2) & 3), V rows of 128 B at c ^ 4*((r >> 1) & 1))
    auto kswz = [](int r) __attribute__((always_inline)) { return D == 128 ? (r >> 1) & 7 : (r >> 2) & 3; };
    auto vswz = [](int r) __attribute__((always_inline)) { return D == 128 ? (r & 3) << 2 : ((r >> 1) & 1) << 2; };
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
    // (the descriptor's fields go through readfirstlane: a descriptor the compiler cannot prove
    // uniform would wrap every DMA instruction in a loop over lanes).  A slice holds nk * BM / BN
    // tiles; the range test is on the tile index, so that the bytes left are not a saturating
    // subtraction, which only the vector unit has.
    const uint32_t slice_tiles = static_cast<uint32_t>(p.nk) * (BM / BN);
    auto tile_rsrc = [&](const uint8_t* base, uint32_t slice, uint32_t rowb, int t) __attribute__((always_inline)) {
        const uint32_t start = static_cast<uint32_t>(t) * BN * rowb;
        const uint32_t left = static_cast<uint32_t>(t) < slice_tiles ? slice - start : 0u;
        const uint64_t addr = uniform_u64(reinterpret_cast<uint64_t>(base) + (left ? start : 0u));
        return make_rsrc(reinterpret_cast<const void*>(addr), static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(left)));
    };
    // tiles past the padded key range read nothing (empty buffer range)
    auto issue_k = [&](int t, uint8_t* slot) __attribute__((always_inline)) {
        const auto r = tile_rsrc(kbase, kslice, KROWB, t);
#pragma unroll
        for (int i = 0; i < KDMA; ++i) buffer_load_lds_b128(r, slot + (wave * KDMA + i) * 1024, kgo[i]);
    };
    auto issue_v = [&](int t, uint8_t* slot) __attribute__((always_inline)) {
        const auto r = tile_rsrc(vbase, vslice, VROWB, t);
#pragma unroll
        for (int i = 0; i < VDMA; ++i) buffer_load_lds_b128(r, slot + (wave * VDMA + i) * 1024, vgo[i]);
    };

    f32x16 oacc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
    float m_run = kNegInf;   // reference max in scaled base-2 units, same in lane and lane^32
    float neg_m = 0.f;       // -m_run, or 0 while m_run = -inf
    float lim = -1.f;        // largest block sum that keeps the reference: kSumLimit, or -1
                             // while m_run = -inf (then every block takes a reference)
    float l_run = 0.f;

    const int kx = kswz(col);
    const int t16 = lane & 15;
    const int vkey_l = half * 4 + (t16 >> 2);
    const int vch_l = ((lane >> 4) & 1) * 16 + 4 * (t16 & 3);

    // ---- S^T = K8 Q8^T for the 32-key block kb of a K tile
    //      (MXFP8: `ke` is the exponent word of this lane's key in block kb)
    //      The lane's two 16-byte chunks per k-step, in Q's channel order (see the Q fragment),
    //      as byte offsets inside a block: the slot and the block then only add an immediate.
    uint32_t koff[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int c0 = (MX ? ks * 4 + half : ks * 4 + half * 2) ^ kx;
        const int c1 = (MX ? ks * 4 + half + 2 : ks * 4 + half * 2 + 1) ^ kx;
        koff[ks][0] = col * KROWB + c0 * 16;
        koff[ks][1] = col * KROWB + c1 * 16;
    }
    // V fragment offsets of the lane per 32-channel block (the key's swizzle depends only on
    // the lane's key inside its group of 8, so the step and block only add an immediate)
    uint32_t voff[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
        const int ch = cb * 32 + vch_l;
        voff[cb] = vkey_l * VROWB + (((ch >> 3) ^ vswz(vkey_l)) * 16) + (ch & 7) * 2;
    }
    // The two K reads of a block's first k-step are issued ahead, at the end of the region B
    // before the region A that multiplies them (as in the bf16 kernel).
    using KPre = u32x4[2];
    auto k_prefetch = [&](const uint8_t* kl, int kb, KPre& pre) __attribute__((always_inline)) {
        const uint8_t* blk = kl + kb * 32 * KROWB;
        pre[0] = *reinterpret_cast<const u32x4*>(blk + koff[0][0]);
        pre[1] = *reinterpret_cast<const u32x4*>(blk + koff[0][1]);
    };
    auto qk_block = [&](const uint8_t* kl, int kb, f32x16& s, uint32_t ke, const KPre& pre) __attribute__((always_inline)) {
        const uint8_t* blk = kl + kb * 32 * KROWB;
        s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 a0 = ks == 0 ? pre[0] : *reinterpret_cast<const u32x4*>(blk + koff[ks][0]);
            const u32x4 a1 = ks == 0 ? pre[1] : *reinterpret_cast<const u32x4*>(blk + koff[ks][1]);
            const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                  (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            if constexpr (MX) {
                // E8M0 of channel block 2ks + half in byte 0: lane half 0 scales the k-step's
                // first 32 channels, lane half 1 the next 32
                const uint32_t sk = ke >> (8 * (2 * ks + half));
                s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s, 0, 0, 0, static_cast<int>(sk), 0,
                                                                    static_cast<int>(qe[ks]));
            } else {
                s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s, 0, 0, 0, 0, 0, 0);
            }
        }
    };
    auto need_mask = [&](int u) __attribute__((always_inline)) {
        const int key0 = u * 32;
        return (key0 + 32 > p.sk) || (CAUSAL && key0 + 31 > wave_row0);
    };
    auto mask_block = [&](int u, f32x16& s) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int key = u * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
            if (key >= p.sk || (CAUSAL && key > my_row)) s[j] = kNegInf;
        }
    };
    // ---- the row's max over a block in scaled base-2 units (c > 0 keeps the order)
    //      (three-operand maxima, which need fewer of the compiler's canonicalising moves than
    //      two-operand ones; c >= FLT_MIN > 0 maps -inf to -inf)
    auto row_max = [&](const f32x16& s, float c) __attribute__((always_inline)) {
        float a = max3(s[0], s[1], s[2]);
        float b = max3(s[8], s[9], s[10]);
        a = max3(a, s[3], s[4]);
        b = max3(b, s[11], s[12]);
        a = max3(a, s[5], s[6]);
        b = max3(b, s[13], s[14]);
        a = max3(a, s[7], s[15]);
        return max_halves(__builtin_fmaxf(a, b)) * c;
    };
    // ---- the reference max (scaled base-2 units): set from a block's scores, moving O and l
    //      to the new reference.  Only the first block of a row and the rare blocks that fail the
    //      check below come here.
    auto rebase = [&](const f32x16& s, float c) __attribute__((always_inline)) {
        const float m_new = fmaxf(m_run, row_max(s, c));
        const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
        m_run = m_new;
        neg_m = m_new == kNegInf ? 0.f : -m_new;
        lim = m_new == kNegInf ? -1.f : kSumLimit;
    };
    // ---- P'^T = exp2(S^T c - m + log2 scale_v) rounded to bf16 for score pairs [lo, hi) of a
    //      block; pair i is word i % 4 of the B operand of 16-key P.V step i / 4
    using PWords = uint32_t[8];
    auto exp_pairs = [&](const f32x16& s, const TileScale& sc, PWords& pw, auto lo_c, auto hi_c)
                         __attribute__((always_inline)) {
        const float bias = neg_m + sc.log2_sv;
#pragma unroll
        for (int i = decltype(lo_c)::value; i < decltype(hi_c)::value; ++i)
            pw[i] = pack_bf16x2(fast_exp2(fmaf(s[2 * i], sc.c, bias)), fast_exp2(fmaf(s[2 * i + 1], sc.c, bias)));
    };
    // ---- this lane's sum of the block's bf16 P' (the values fed to P.V)
    auto block_sum = [&](const PWords& pw) __attribute__((always_inline)) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = add_bf16_pair(pw[i], a);
        return a;
    };
    // ---- a block whose exponentials ran against the reference max: its sum of probabilities
    //      (P' back to unscaled ones); above the limit on any lane (some probability above 2^8, or
    //      a row without a reference yet) the block takes its own max as the reference and its
    //      exponentials rerun.  Then the sum joins l.
    auto settle = [&](const f32x16& s, const TileScale& sc, PWords& pw, float raw) __attribute__((always_inline)) {
        float bs = raw * sc.inv_sv;
        if (__any(bs > lim)) {
            rebase(s, sc.c);
            exp_pairs(s, sc, pw, IC<0>{}, IC<8>{});
            bs = block_sum(pw) * sc.inv_sv;
        }
        l_run += bs;
    };
    // ---- O^T += V^T P'^T over the 32-key block kb of a V tile (transposing reads)
    auto pv_block = [&](const uint8_t* vl, int kb, const PWords& pw) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const auto b = __builtin_bit_cast(bf16x8, u32x4{pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]});
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) {
                u32x2 part[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int key0 = kb * 32 + ks * 16 + r * 8;   // multiple of 8: same swizzle
                    part[r] = lds_read_tr16_b64(vl + key0 * VROWB + voff[cb]);
                }
                const auto a = __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
                oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, oacc[cb], 0, 0, 0);
            }
        }
    };

    // Score pairs of block u + 1 (of 8 per lane) whose exponentials run under block u's P.V
    // MFMAs; the rest and the block sum run under the S MFMAs of block u + 2, where the block is
    // settled.  EARLY = 8 runs all of it, sum included, under P.V and settles the block right
    // after.
    constexpr bool NARROW = EARLY == 8;
    using Early = IC<EARLY>;
    constexpr int VALU_A = NARROW ? 0 : 5 * (8 - EARLY) + 8;
    constexpr int PV_MFMA = 2 * CBLK;
    constexpr int VALU_B = 5 * EARLY + (NARROW ? 8 : 0);
    constexpr int WAIT_VM0 = 0x0F70;                // s_waitcnt vmcnt(0)
    constexpr int VM_PROLOGUE = VDMA + KDMA;        // V_0 and K_1 may still be in flight
    static_assert(VM_PROLOGUE < 16, "vmcnt immediate");
    constexpr int WAIT_K0 = VM_PROLOGUE | 0x0F70;
    // region A: S of the next block (D/64 fp8 MFMAs, two K reads each); unless NARROW also the last
    //           exponentials of the current block and its raw sum, which it returns
    auto region_a = [&](const uint8_t* kl, int kb, uint32_t ke, f32x16& sn, const f32x16& s, const TileScale& sc,
                        PWords& pw, const KPre& pre) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        qk_block(kl, kb, sn, ke, pre);
        float raw = 0.f;
        if constexpr (!NARROW) {
            exp_pairs(s, sc, pw, Early{}, IC<8>{});
            raw = block_sum(pw);
            // keep the sum here: without a use inside the region the compiler would sink it
            asm volatile("" ::"v"(raw));
        }
        // the later k-steps' reads open the region, under the first MFMA
        sched_region<KS, 2 * (KS - 1), 2 * (KS - 1), 1, VALU_A, 0>(std::make_integer_sequence<int, KS>{});
        __builtin_amdgcn_sched_barrier(0);
        return raw;
    };
    // region B: P.V of the current block under the first exponentials of the next one (NARROW: all
    // of them and their raw sum, which it returns); with PRE, it also reads the first k-step of the
    // next region A's K block
    auto region_b = [&](const uint8_t* vl, int kb, const PWords& pw, const f32x16& sn, const TileScale& sc_n,
                        PWords& pw_next, auto vmem_c, auto pre_c, const uint8_t* kl_next, int kb_next,
                        KPre& pre) __attribute__((always_inline)) {
        constexpr int NPRE = decltype(pre_c)::value ? 2 : 0;
        pv_block(vl, kb, pw);
        exp_pairs(sn, sc_n, pw_next, IC<0>{}, Early{});
        float raw = 0.f;
        if constexpr (NARROW) {
            raw = block_sum(pw_next);
            asm volatile("" ::"v"(raw));
        } else {
            // keep the exponentials here: without a use inside the region the compiler would sink
            // them to the region that consumes them
#pragma unroll
            for (int i = 0; i < EARLY; ++i) asm volatile("" ::"v"(pw_next[i]));
        }
        if constexpr (NPRE > 0) k_prefetch(kl_next, kb_next, pre);
        sched_region<PV_MFMA, 2 * PV_MFMA + NPRE, 2 * CBLK, 2, VALU_B, decltype(vmem_c)::value>(
            std::make_integer_sequence<int, PV_MFMA>{});
        __builtin_amdgcn_sched_barrier(0);
        return raw;
    };

    // ---- main loop over 64-key tiles, software-pipelined over their 32-key blocks (as in the
    //      bf16 kernel).  Tile t's K sits in k slot t%2 and its V in v slot t%2; even blocks keep
    //      their scores in s0 and probabilities in p0, odd ones in s1 / p1.  The barrier of
    //      iteration t guarantees that every wave's part of V_t and K_{t+1} has landed and that no
    //      wave still reads K_t or V_{t-1}: their slots then take K_{t+2}, V_{t+1}.
    using NoVmem = IC<0>;
    using DmaVmem = IC<KDMA + VDMA + (MX ? 2 : 0)>;
    // (MXFP8: ke[0] holds the exponent words of tile t, ke[1] those of tile t+1; the words of
    // tile t+2 are loaded with its K tile)
    using Pre = std::true_type;
    using NoPre = std::false_type;
    auto iteration = [&](int t, auto par_c, f32x16& s0, f32x16& s1, PWords& p0, PWords& p1, TileScale& sc,
                         u32x2 (&ke)[2], KPre& pre) __attribute__((always_inline)) {
        using Cur = IC<decltype(par_c)::value>;
        using Nxt = IC<decltype(par_c)::value ^ 1>;
        const TileScale sc_next = tile_scale(t + 1);
        // block 2t (s0, p0) with the S of block 2t+1 (into s1)
        float raw = region_a(k_slot(Cur{}), 1, ke[0][1], s1, s0, sc, p0, pre);
        if (need_mask(2 * t + 1)) mask_block(2 * t + 1, s1);
        if constexpr (!NARROW) settle(s0, sc, p0, raw);
        __builtin_amdgcn_s_waitcnt(WAIT_VM0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        u32x2 ke_new = {0u, 0u};
        if constexpr (MX) ke_new = kexp_load(t + 2);
        issue_k(t + 2, k_slot(Cur{}));
        issue_v(t + 1, v_slot(Nxt{}));
        raw = region_b(v_slot(Cur{}), 0, p0, s1, sc, p1, DmaVmem{}, Pre{}, k_slot(Nxt{}), 0, pre);
        if constexpr (NARROW) settle(s1, sc, p1, raw);
        // block 2t+1 (s1, p1) with the S of block 2t+2, the first block of the next tile (into s0)
        raw = region_a(k_slot(Nxt{}), 0, ke[1][0], s0, s1, sc, p1, pre);
        if (need_mask(2 * t + 2)) mask_block(2 * t + 2, s0);
        if constexpr (!NARROW) settle(s1, sc, p1, raw);
        __builtin_amdgcn_sched_barrier(0);
        // the next region A (an iteration or the last tile) starts on block 1 of K_{t+1}
        raw = region_b(v_slot(Cur{}), 1, p1, s0, sc_next, p0, NoVmem{}, Pre{}, k_slot(Nxt{}), 1, pre);
        if constexpr (NARROW) settle(s0, sc_next, p0, raw);
        sc = sc_next;
        ke[0] = ke[1];
        ke[1] = ke_new;
    };
    // the last tile: its two blocks, nothing further to load
    auto last = [&](int t, auto par_c, const f32x16& s0, f32x16& s1, PWords& p0, PWords& p1, const TileScale& sc,
                    const u32x2 (&ke)[2], KPre& pre) __attribute__((always_inline)) {
        using Cur = IC<decltype(par_c)::value>;
        float raw = region_a(k_slot(Cur{}), 1, ke[0][1], s1, s0, sc, p0, pre);
        if (need_mask(2 * t + 1)) mask_block(2 * t + 1, s1);
        if constexpr (!NARROW) settle(s0, sc, p0, raw);
        __builtin_amdgcn_s_waitcnt(WAIT_VM0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        raw = region_b(v_slot(Cur{}), 0, p0, s1, sc, p1, NoVmem{}, NoPre{}, nullptr, 0, pre);
        if constexpr (!NARROW) {
            exp_pairs(s1, sc, p1, Early{}, IC<8>{});
            raw = block_sum(p1);
        }
        settle(s1, sc, p1, raw);
        pv_block(v_slot(Cur{}), 1, p1);
    };

    if (ntiles > 0) {
        using Zero = IC<0>;
        using One = IC<1>;
        u32x2 ke[2] = {{0u, 0u}, {0u, 0u}};
        if constexpr (MX) {   // issued before the DMA, so the wait below covers them too
            ke[0] = kexp_load(0);
            ke[1] = kexp_load(1);
        }
        // the first tile's block scales are requested with its K/V, not after the barrier below
        // (a fence: loads stay behind it), which would add a round trip before the first scores
        TileScale sc = tile_scale(0);
        issue_k(0, k_slot(Zero{}));
        issue_v(0, v_slot(Zero{}));
        issue_k(1, k_slot(One{}));
        __builtin_amdgcn_s_waitcnt(WAIT_K0);   // this wave's part of K_0 has landed
        __syncthreads();
        f32x16 s0, s1;
        PWords p0, p1;
        KPre pre;
        k_prefetch(k_slot(Zero{}), 0, pre);
        qk_block(k_slot(Zero{}), 0, s0, ke[0][0], pre);
        if (need_mask(0)) mask_block(0, s0);
        rebase(s0, sc.c);                     // the row's first reference max
        exp_pairs(s0, sc, p0, IC<0>{}, Early{});
        if constexpr (NARROW) l_run = block_sum(p0) * sc.inv_sv;
        k_prefetch(k_slot(Zero{}), 1, pre);   // the first region A starts on block 1 of K_0
        // Tiles up to `need` hold a key that some row of this wave sees; past them (the diagonal
        // tiles of the rows above) the wave only keeps the ring's waits, barriers and its share
        // of the DMA.  Wave-uniform.
        int need = ntiles;
        if constexpr (CAUSAL) need = min(ntiles, (wave_row0 + 31) / BN + 1);
        const int e = min(need, ntiles - 1);   // tiles run through iteration()
        int t = 0;
        for (; t + 2 <= e; t += 2) {
            iteration(t, Zero{}, s0, s1, p0, p1, sc, ke, pre);
            iteration(t + 1, One{}, s0, s1, p0, p1, sc, ke, pre);
        }
        const bool odd = t < e;
        if (odd) iteration(t++, Zero{}, s0, s1, p0, p1, sc, ke, pre);
        if (need == ntiles) {
            if (odd) last(t, One{}, s0, s1, p0, p1, sc, ke, pre);
            else last(t, Zero{}, s0, s1, p0, p1, sc, ke, pre);
        } else {
            // tile t has parity t & 1; the last tile issues no further DMA
            auto drain = [&](int u, auto par_c) __attribute__((always_inline)) {
                using Cur = IC<decltype(par_c)::value>;
                using Nxt = IC<decltype(par_c)::value ^ 1>;
                __builtin_amdgcn_s_waitcnt(WAIT_VM0);
                __syncthreads();
                if (u + 1 < ntiles) {
                    issue_k(u + 2, k_slot(Cur{}));
                    issue_v(u + 1, v_slot(Nxt{}));
                }
            };
            bool par = odd;
            for (; t < ntiles; ++t) {
                if (par) drain(t, One{});
                else drain(t, Zero{});
                par = !par;
            }
        }
    }

    const float l_tot = l_run + swap_halves(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (my_row < p.sq) {
        uint16_t* orow = static_cast<uint16_t*>(p.o) + (bb * p.ov.sb + h * p.ov.sh + my_row * p.ov.ss);
        store_o_row<CBLK>(orow, oacc, inv, half);
        if (p.lse != nullptr && half == 0) {
            const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;   // m_run is scaled
            p.lse[(static_cast<int64_t>(bb) * p.hq + h) * p.sq + my_row] = lse;
        }
    }
    }
    if constexpr (CAUSAL) {
        // the pair's light block: the slots are rewritten only after every wave is done
        if (mblk != mrev) {
            mblk = mrev;
            __syncthreads();
            goto next_item;
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const Fp8AttnParams& p, int d, bool causal, hipStream_t stream) {
    if (d != 64 && d != 128) return hipErrorInvalidValue;
    // causal grids pair query blocks n-1-j and j in one workgroup
    const int64_t nwg = static_cast<int64_t>(p.b) * p.hq * (causal ? (p.n_mblocks + 1) / 2 : p.n_mblocks);
    if (nwg == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(nwg));
    const bool mx = p.q_exps != nullptr;
    // non-causal d128: two query blocks per workgroup when that grid still fills the device
    if (d == 128 && !causal && MHA_FP8_BLOCKS_PER_WG > 1) {
        constexpr int R = MHA_FP8_BLOCKS_PER_WG;
        const int64_t nwg_r = static_cast<int64_t>(p.b) * p.hq * ((p.n_mblocks + R - 1) / R);
        const auto kernel = mx ? attn_fwd_fp8_kernel<128, false, true, R> : attn_fwd_fp8_kernel<128, false, false, R>;
        int groups = 0;
        const hipError_t e = resident_groups(reinterpret_cast<const void*>(kernel), NTHREADS * R, &groups);
        if (e != hipSuccess) return e;
        if (nwg_r >= groups) {
            hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(nwg_r)), dim3(NTHREADS * R), 0, stream, p);
            return hipGetLastError();
        }
    }
    auto go = [&](auto d_c) {
        constexpr int DD = decltype(d_c)::value;
        if (mx && causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<DD, true, true>), grid, dim3(NTHREADS), 0, stream, p);
        if (mx && !causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<DD, false, true>), grid, dim3(NTHREADS), 0, stream, p);
        if (!mx && causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<DD, true, false>), grid, dim3(NTHREADS), 0, stream, p);
        if (!mx && !causal)
            hipLaunchKernelGGL((attn_fwd_fp8_kernel<DD, false, false>), grid, dim3(NTHREADS), 0, stream, p);
    };
    if (d == 128)
        go(std::integral_constant<int, 128>{});
    else
        go(std::integral_constant<int, 64>{});
    return hipGetLastError();
}

}  // namespace mha
