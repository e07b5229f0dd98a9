// Fused attention forward, bf16 in / bf16 out, fp32 accumulation, for gfx950.
//
// Computes O = softmax(scale * Q K^T + causal mask) V and the natural-log LSE per
// row: the MHA forward pass tuned on "Tune MHA config & small-head pipeline
// pathology" (Motivation; Technical Details: head-dim buckets 64, 128 and the
// dqk=192/dv=128 "pe" bucket; Profile 2: pipelining depth as the main lever).
//
// Work decomposition: one workgroup per (batch, query head, block of BM query
// rows), one wave per 32 rows; causal grids give each workgroup the pair of
// blocks j and n-1-j instead (packed sequences only on short grids).  The kernel computes the TRANSPOSED scores
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every lane holds one query row
// (lane % 32) and half of the keys of each 32-key block: the row max and row sum
// stay in the lane except for one exchange with lane ^ 32, and the probabilities
// P^T are already laid out as the B operand of O^T = V^T P^T (the key order
// inside one 16-key MFMA step is permuted the same way on both operands, which
// leaves the contraction unchanged).
//
//   Q      32 rows x d_qk per wave, loaded once into registers (B operand).
//   K, V   BN-key tiles stream global -> LDS by DMA (buffer_load ... lds) into two
//          rings of two slots each, rows unpadded and 16-byte chunks XOR-swizzled
//          for conflict-free reads: K rows feed the A operand of S^T with one
//          ds_read_b128 per MFMA, V rows feed the A operand of O^T through
//          transposing reads (ds_read_b64_tr_b16).
//   loop   software-pipelined across 32-key blocks: the S MFMAs of block u+1
//          run under the last exponentials of block u and its row sum, the P.V
//          MFMAs of block u under the first exponentials of block u+1.  The
//          instruction interleaving is fixed with scheduling group barriers, and
//          the DMA of later tiles is spread over the MFMA stream so no wave stalls
//          on a full address queue.
//   causal key tiles past the block's last row are never loaded; masking is
//          applied only on tiles that cross the diagonal or the ragged end, by
//          setting the score to -inf, which the exponential maps to exactly 0.
//   softmax online, in base 2: p = exp2(s*c - m*c) with c = |scale| * log2 e
//          (at least FLT_MIN, so that a zero scale still maps -inf to 0) folded
//          into one FMA (a negative scale negates Q, which is exact).  m is a
//          reference max, not the running one: a row takes the max of its first
//          block, and each later block's exponentials run against the reference
//          as it stands.  The block's sum of probabilities, which the row sum
//          needs anyway, then checks it: at most 2^8 per lane means no
//          probability above 2^8 (the reference lags the row max by at most 8 in
//          log2 units, as a lazy rescale would keep it); above, the block takes
//          its own max as the new reference, O and l are rescaled and the block's
//          exponentials rerun.  No per-block max is taken on the common path.
//          The row sum adds the bf16-rounded probabilities that enter P.V
//          (v_dot2_f32_bf16), so O is normalised by exactly the weights it was
//          built from.
//
// Every global load goes through a buffer resource clamped to the (batch, head)
// slice, so rows past sq / sk read as zero instead of faulting.

#include <algorithm>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "kernels.h"

namespace mha {
namespace {

// A lane's sum of the 16 rounded probabilities of a block it computed against the reference max;
// at most this, each probability is at most 2^8 (the reference lags the row max by at most 8 in
// log2 units), otherwise the block takes a new reference.
constexpr float kSumLimit = 256.0f;
template <int N> using IC = std::integral_constant<int, N>;
constexpr float kMinScale = 1.17549435e-38f;   // FLT_MIN

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kGrpValu = 0x002, kGrpMfma = 0x008, kGrpVmem = 0x010, kGrpDsRead = 0x100;

// One slot of an interleaved region: one MFMA, then (while slots last) one VMEM
// instruction, DS_PER LDS reads and VALU_PER vector ALU instructions.
template <int I, int VMEM, int DS_SLOTS, int DS_PER, int VALU_SLOTS, int VALU_PER>
__device__ __forceinline__ void sched_slot() {
    __builtin_amdgcn_sched_group_barrier(kGrpMfma, 1, 0);
    if constexpr (I < VMEM) __builtin_amdgcn_sched_group_barrier(kGrpVmem, 1, 0);
    if constexpr (I < DS_SLOTS) __builtin_amdgcn_sched_group_barrier(kGrpDsRead, DS_PER, 0);
    if constexpr (I < VALU_SLOTS) __builtin_amdgcn_sched_group_barrier(kGrpValu, VALU_PER, 0);
}

// Scheduling pattern of a region with MFMAS matrix instructions fed by DS reads: DS_PRE
// reads go first (the operands of the first MFMAs), the other DS_TOTAL - DS_PRE follow
// DS_PER per MFMA, VMEM instructions go one per MFMA, and VALU instructions are spread
// evenly over the MFMAs.
template <int MFMAS, int DS_TOTAL, int DS_PRE, int DS_PER, int VALU, int VMEM, int... I>
__device__ __forceinline__ void sched_region(std::integer_sequence<int, I...>) {
    constexpr int DS_SLOTS = (DS_TOTAL - DS_PRE) / DS_PER;
    constexpr int VALU_PER = (VALU + MFMAS - 1) / MFMAS;
    constexpr int VALU_DIV = VALU_PER > 0 ? VALU_PER : 1;
    constexpr int VALU_SLOTS = VALU_PER > 0 ? (VALU + VALU_DIV - 1) / VALU_DIV : 0;
    if constexpr (DS_PRE > 0) __builtin_amdgcn_sched_group_barrier(kGrpDsRead, DS_PRE, 0);
    (sched_slot<I, VMEM, DS_SLOTS, DS_PER, VALU_SLOTS, VALU_PER>(), ...);
}

// Tile shape per head-dim pair: BM query rows per workgroup (32 per wave), BN keys per tile.
// 128-row workgroups run two (d128) to four (d32) per CU; the 256-row one runs alone with 8
// waves, which halves the K/V traffic per FLOP of the wide d192/d128 tiles.
// EARLY: score pairs (of the 8 per lane and block) of block u+1 whose exponentials run under the
// P.V MFMAs of block u; the other pairs, the block sum and its check run under the S MFMAs of
// block u+2.  The wide heads split the VALU work between the two regions about as their MFMAs
// split; the narrow ones, whose P.V and S regions are short, put all of it under P.V, which also
// keeps d64 within 168 VGPRs (three workgroups per CU).
#ifndef MHA_EARLY_WIDE
#define MHA_EARLY_WIDE 4
#endif
// Query heads per workgroup for d128 under GQA (see HPW below); 1 turns it off
#ifndef MHA_HEADS_PER_WG
#define MHA_HEADS_PER_WG 2
#endif
// REV: causal blocks in the lower half of their sequence run their key tiles downward (see the
// main loop), for the head dims whose K/V per head outgrows an XCD's 4 MiB L2 on long sequences
// (d192/d128: 5.2 MB at 8192 keys); the GQA shapes of the narrower heads share one kv head's K/V
// between several query heads and keep it in L2 either way.
template <int DQK, int DV> struct TileCfg;
template <> struct TileCfg<32, 32> { static constexpr int BM = 128, BN = 64, EARLY = 8; static constexpr bool REV = false; };
template <> struct TileCfg<64, 64> { static constexpr int BM = 128, BN = 64, EARLY = 8; static constexpr bool REV = false; };
template <> struct TileCfg<128, 128> { static constexpr int BM = 128, BN = 64, EARLY = MHA_EARLY_WIDE; static constexpr bool REV = false; };
template <> struct TileCfg<192, 128> { static constexpr int BM = 256, BN = 64, EARLY = MHA_EARLY_WIDE; static constexpr bool REV = true; };

// Key tiles of causal query block m (keys [0, min(sk, (m + 1) BM))).
template <int BM, int BN>
__host__ __device__ __forceinline__ int split_causal_tiles(int m, int sk) {
    const int64_t keys = static_cast<int64_t>(m + 1) * BM < sk ? static_cast<int64_t>(m + 1) * BM : sk;
    return static_cast<int>((keys + BN - 1) / BN);
}

// EXT: sliding window (keys j with i - window_left <= j <= i + window_right, positions inside
// the sequence) and per-head sink logits.  SPLIT: grids that would underfill the device give each
// query block (non-causal) or each pair of causal blocks (n-1-j, j) p.n_split workgroups, each
// over one contiguous range of the key tiles, which leave partial states for attn_split_merge.
// HPW: query heads per workgroup.  Under GQA the query heads of one kv head read the same K/V
// tiles; a workgroup of HPW x (BM / 32) waves takes the same BM rows of HPW such heads, so each
// tile that the DMA brings into LDS serves HPW times the rows (each wave's rows, diagonal and
// registers stay as with one head).  Not with the key split; with windows and sinks only where
// no left window is set (the launcher decides).
template <int DQK, int DV, bool CAUSAL, bool VARLEN, bool PAIRED, bool EXT, bool SPLIT, int HPW = 1>
// Windows and sinks at d64 run four workgroups per CU (128 VGPRs): a 128-token window gives a
// workgroup a few tiles, so the grid is bound by latency more than by issue (measured: the
// GPT-OSS-like window layer 78.6 -> 71.9 us; the full causal layer with sinks unchanged; the
// paired d64 kernel spills in its loop at 128 VGPRs and loses 13%, so it keeps three).
__global__ __launch_bounds__((TileCfg<DQK, DV>::BM * 2 * HPW), (EXT && DQK <= 64 ? 4 : HPW > 1 ? 1 : 2)) void attn_fwd_bf16_kernel(const AttnParams p) {
    constexpr int BM = TileCfg<DQK, DV>::BM;           // query rows per head and workgroup
    constexpr int RWAVES = BM / 32;                    // one wave per 32 rows of a head
    constexpr int NTHREADS = BM * 2 * HPW;
    constexpr int NWAVES = NTHREADS / 64;
    static_assert(HPW == 1 || !SPLIT, "several heads per workgroup without the key split");
    constexpr int BN = TileCfg<DQK, DV>::BN;           // keys per tile
    constexpr int KROWB = DQK * 2;            // bytes per K row in LDS (16-byte chunks XOR-swizzled)
    constexpr int VROWB = DV * 2;             // bytes per V row in LDS (row-major, swizzled)
    constexpr int KTILE = BN * KROWB;
    constexpr int VTILE = BN * VROWB;
    constexpr int KDMA = KTILE / 1024 / NWAVES;   // 1 KiB DMA blocks per wave per K tile
    constexpr int VDMA = VTILE / 1024 / NWAVES;
    constexpr int KSTEPS = DQK / 16;          // MFMA k-steps for S^T
    constexpr int CBLK = DV / 32;             // 32-channel output blocks
    static_assert(BN == 64, "the loop pipelines the two 32-key blocks of a tile");
    static_assert(KDMA * NWAVES * 1024 == KTILE && VDMA * NWAVES * 1024 == VTILE, "DMA blocks must cover the tiles");
    static_assert(2 * (KTILE + VTILE) <= (BM == 128 ? 80 : 160) * 1024, "the workgroups of a CU must fit in LDS");

    // Two slots per ring, each a distinct LDS object: the compiler's wait insertion then
    // knows that the DMA filling one slot cannot alias the fragment reads of another.
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
    //      Causal attention on a grid of a few rounds pairs the query blocks of a head
    //      (PAIRED): a workgroup takes block n-1-j and then block j, so every workgroup does
    //      the same work and the grid has no tail of light workgroups.
    static_assert(CAUSAL || !PAIRED, "only causal blocks differ in work");
    static_assert(!EXT || !PAIRED, "windows and sinks run on unpaired grids");
    static_assert(!SPLIT || (!VARLEN && !EXT && CAUSAL == PAIRED), "the key split runs on dense grids, paired when causal");
    const int nwg = gridDim.x;
    const int nwg8 = nwg & ~7;
    const int pid = blockIdx.x;
    const int per_head = PAIRED ? (p.n_mblocks + 1) / 2 : p.n_mblocks;
    int lid = pid < nwg8 ? (pid & 7) * (nwg8 >> 3) + (pid >> 3) : pid;
    if constexpr (VARLEN) {
        // Packed sequences differ in length, so contiguous eighths of the grid would give the
        // XCDs very different work.  Deal (sequence, kv head) units round-robin instead: XCD x
        // takes units x, x + 8, ... (every sequence, one kv head in eight, with its query heads
        // and blocks kept together); units past the last full round of 8 keep their own ids.
        const int unit = per_head * (p.group / HPW);         // workgroups per (sequence, kv head)
        const int full = (nwg / unit / 8) * 8 * unit;
        if (pid < full) {
            const int i = pid >> 3;
            lid = ((pid & 7) + 8 * (i / unit)) * unit + i % unit;
        } else {
            lid = pid;
        }
    }
    // SPLIT: the key ranges of one query block (or pair) are consecutive ids (one XCD), range fastest
    const int split = SPLIT ? lid % p.n_split : 0;
    if constexpr (SPLIT) lid /= p.n_split;
    [[maybe_unused]] const int item = lid;    // (batch, head, query block or pair) of this workgroup
    const int mrev = lid % per_head;
    const int bh = lid / per_head;
    int mblk = CAUSAL ? (p.n_mblocks - 1 - mrev) : mrev;   // causal: heavy blocks first
    // SPLIT && CAUSAL: the pair's key tiles, block n-1-j's then block j's, in one sequence of
    // L = LA + LB tiles; this workgroup takes tiles [a, b) of it, as the tail [a, min(b, LA)) of
    // the first block and, if b > LA, the head [0, b - LA) of the second.  `which` is the block
    // in hand (0: n-1-j, 1: j) and [seg0, seg1) its tiles.
    [[maybe_unused]] int which = 0, seg0 = 0, seg1 = 0, pair_la = 0, pair_lb = 0, pair_b = 0;
    if constexpr (SPLIT && CAUSAL) {
        const int ma = p.n_mblocks - 1 - mrev;
        pair_la = split_causal_tiles<BM, BN>(ma, p.sk);
        pair_lb = ma != mrev ? split_causal_tiles<BM, BN>(mrev, p.sk) : 0;
        const int len = pair_la + pair_lb;
        const int a = split * len / p.n_split;
        pair_b = (split + 1) * len / p.n_split;
        if (a < pair_la) {
            seg0 = a;
            seg1 = min(pair_b, pair_la);
        } else {
            mblk = mrev;
            which = 1;
            seg0 = a - pair_la;
            seg1 = pair_b - pair_la;
        }
    }
    bool lds_zeroed = false;
next_item:
    // A pair's second block passes the lane index through an empty asm statement: nothing
    // derived from it (fragment addresses, mask offsets) is then hoisted out of the loop over
    // the pair, where it would stay live across every tile and crowd the tile loop's registers.
    int tid = threadIdx.x;
    if constexpr (PAIRED) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31;     // query column of this lane in S^T / O^T
    const int half = lane >> 5;    // which half of the wave
    {
        // bh: (batch, head) or, with HPW > 1, (batch, group of HPW heads); the wave's head
        const int h = HPW == 1 ? bh % p.hq : (bh % (p.hq / HPW)) * HPW + wave / RWAVES;
        const int bb = HPW == 1 ? bh / p.hq : bh / (p.hq / HPW);
        const int g = h / p.group;   // the same for every wave: HPW divides the group

        // ---- this workgroup's sequence: the whole batch row, or (varlen) packed tokens
        //      [q0, q0 + sq) and [k0, k0 + sk) of the token axis.  Offsets are clamped to the
        //      packed extent and the lengths to the declared maxima, so inconsistent offsets
        //      can give wrong values but no access outside the tensors.
        int sq = p.sq, sk = p.sk;
        int64_t qrow0 = static_cast<int64_t>(bb) * p.qv.sb, krow0 = static_cast<int64_t>(bb) * p.kv.sb;
        int64_t vrow0 = static_cast<int64_t>(bb) * p.vv.sb, orow0 = static_cast<int64_t>(bb) * p.ov.sb;
        int64_t lse0 = (static_cast<int64_t>(bb) * p.hq + h) * p.sq;
        uint32_t qslice = p.qv.slice_bytes, kslice = p.kv.slice_bytes, vslice = p.vv.slice_bytes;
        if constexpr (VARLEN) {
            const int qa = min(max(p.cu_q[bb], 0), p.total_q);
            const int qe = min(max(p.cu_q[bb + 1], qa), p.total_q);
            const int ka = min(max(p.cu_k[bb], 0), p.total_k);
            const int ke = min(max(p.cu_k[bb + 1], ka), p.total_k);
            sq = min(qe - qa, p.sq);
            sk = min(ke - ka, p.sk);
            if (mblk * BM >= sq) {      // the whole workgroup: past this sequence's rows
                if constexpr (PAIRED) goto item_done;
                else return;
            }
            qrow0 = static_cast<int64_t>(qa) * p.qv.ss;
            orow0 = static_cast<int64_t>(qa) * p.ov.ss;
            krow0 = static_cast<int64_t>(ka) * p.kv.ss;
            vrow0 = static_cast<int64_t>(ka) * p.vv.ss;
            lse0 = static_cast<int64_t>(h) * p.total_q + qa;
            qslice = static_cast<uint32_t>((static_cast<int64_t>(sq - 1) * p.qv.ss + DQK) * 2);
            kslice = sk > 0 ? static_cast<uint32_t>((static_cast<int64_t>(sk - 1) * p.kv.ss + DQK) * 2) : 0u;
            vslice = sk > 0 ? static_cast<uint32_t>((static_cast<int64_t>(sk - 1) * p.vv.ss + DV) * 2) : 0u;
        }
        const char* qbase = static_cast<const char*>(p.q) + 2 * (qrow0 + h * p.qv.sh);
        const char* kbase = static_cast<const char*>(p.k) + 2 * (krow0 + g * p.kv.sh);
        const char* vbase = static_cast<const char*>(p.v) + 2 * (vrow0 + g * p.vv.sh);
        const auto qrs = make_rsrc(qbase, qslice);

        const int wave_row0 = mblk * BM + (HPW == 1 ? wave : wave % RWAVES) * 32;
        const int my_row = wave_row0 + col;

        // ---- Q fragment (B operand of S^T = K Q^T): lane holds Q[my_row][kk*16 + half*8 .. +8]
        bf16x8 qf[KSTEPS];
        {
            const uint32_t rowoff = my_row < sq ? static_cast<uint32_t>(my_row * p.qv.ss * 2) : kOutOfRange;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const uint32_t off = rowoff == kOutOfRange ? kOutOfRange : rowoff + (kk * 16 + half * 8) * 2;
                qf[kk] = __builtin_bit_cast(bf16x8, buffer_load_b128(qrs, off));
            }
        }
        const float c = fmaxf(fabsf(p.scale_log2), kMinScale);   // base-2 score scale, > 0

        int kv_end = CAUSAL ? min(sk, (mblk + 1) * BM) : sk;
        int t0 = 0;   // first key tile: keys left of every row's window are never loaded
        if constexpr (EXT) {
            if (!CAUSAL && p.window_right >= 0) kv_end = min(sk, (mblk + 1) * BM + p.window_right);
            if (p.window_left >= 0) t0 = max(0, mblk * BM - p.window_left) / BN;
        }
        if constexpr (SPLIT) {
            // key tiles [t0, t1): non-causal, range `split` of the ceil(sk / BN) tiles (the ranges
            // differ by at most one tile); causal, the segment of the block in hand.  The K and V
            // slices end at the range, so the DMA that runs ahead of the last tile reads nothing
            // past it.
            if constexpr (CAUSAL) {
                t0 = seg0;
                kv_end = min(kv_end, seg1 * BN);
            } else {
                const int nt = (sk + BN - 1) / BN;
                t0 = split * nt / p.n_split;
                kv_end = min(sk, (split + 1) * nt / p.n_split * BN);
            }
            if (kv_end < sk) {
                kslice = static_cast<uint32_t>((static_cast<int64_t>(kv_end - 1) * p.kv.ss + DQK) * 2);
                vslice = static_cast<uint32_t>((static_cast<int64_t>(kv_end - 1) * p.vv.ss + DV) * 2);
            }
        }
        const int ntiles = (kv_end + BN - 1) / BN;
        // The loop runs over positions t0, t0 + 1, ... of the tile sequence.  With REV, causal
        // blocks in the lower half of their sequence (block m with m < n - 1 - m, n blocks: the
        // light block of each pair (n-1-j, j)) take their tiles downward, from the diagonal to
        // tile t0 = 0.  The pairs of a head start together on one XCD: all of them read tile tau
        // on the way up and tile L + 1 - tau on the way down (L + 2 tiles per pair), so the L2
        // keeps the K/V tiles they share instead of each pair restarting at tile 0 at its own
        // time.  The direction depends on the block and its sequence alone, so packed and dense
        // calls, paired or not, sum every row in the same order.  Downward, position t is tile
        // ntiles - 1 - t = (t ^ -1) + ntiles, and positions past the last tile map to negative
        // tiles, whose buffer range is empty (tile_rsrc); block u of the positions is block
        // (u ^ -2) + 2 ntiles of the key axis.
        constexpr bool CAN_REV = TileCfg<DQK, DV>::REV && CAUSAL && !EXT && !SPLIT;
        const bool rev = CAN_REV && mblk < (sq + BM - 1) / BM - 1 - mblk;
        const int rev_x = rev ? -1 : 0, rev_c = rev ? ntiles : 0;
        auto tile_at = [&](int t) __attribute__((always_inline)) {
            if constexpr (!CAN_REV) return t;
            else return (t ^ rev_x) + rev_c;
        };
        auto blk_at = [&](int u) __attribute__((always_inline)) {
            if constexpr (!CAN_REV) return u;
            else return (u ^ (rev_x * 2)) + rev_c * 2;
        };

        // ---- DMA: lane l of a wave writes 16 bytes at block base + 16*l, and its global
        //      address decides what lands there.  The 16-byte chunks of a row are XOR-swizzled
        //      so that the fragment reads are bank-conflict free on gfx950's LDS, which serves
        //      256 bytes per clock (16 lanes of a b128 read, 32 lanes of a b64 read):
        //        K: the 16 rows one b128 read touches land on 16 distinct 16-byte bank groups;
        //        V: the 4 rows one transposing read touches land on 4 distinct 64-byte quarters.
        //      The per-lane global offsets are loop-invariant; each tile's buffer descriptor is
        //      based at the tile and bounded by the slice, so keys past sk land as zeros.
        auto kswz = [](int r) __attribute__((always_inline)) {
            // rows of 256 B; of 64 B (4 chunks: the 16 rows of a read fall on 4 row pairs mod 4);
            // else 128/384 B
            return KROWB % 256 == 0 ? (r & 15) : KROWB == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7);
        };
        auto vswz = [](int r) __attribute__((always_inline)) {
            // 64-B rows: the 4 keys a transposing read touches are 256 contiguous bytes already
            return VROWB % 256 == 0 ? ((r & 3) << 2) : VROWB == 64 ? 0 : (((r >> 1) & 1) << 2);
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
        // A tile's buffer: its byte offset into the slice and the bytes left after it.  Per item,
        // the number of tiles that start inside a slice (a slice holds less than 4 GiB) and the
        // tile stride; tile t < that number then starts at t * stride < 2^32, so the loop needs
        // 32-bit scalar arithmetic only (the scalar unit has no unsigned 64-bit less-than).  A
        // tile index is taken as unsigned: the negative ones of a downward block (CAN_REV) start
        // past any slice.
        auto tile_geom = [](const View& vw, uint32_t slice, uint32_t& stride, uint32_t& tiles) __attribute__((always_inline)) {
            const uint64_t b = static_cast<uint64_t>(BN * 2) * static_cast<uint64_t>(vw.ss);
            stride = static_cast<uint32_t>(b);
            tiles = slice == 0 ? 0u : b >= slice ? 1u : (slice - 1) / stride + 1;
        };
        uint32_t kstride, ktiles, vstride, vtiles;
        tile_geom(p.kv, kslice, kstride, ktiles);
        tile_geom(p.vv, vslice, vstride, vtiles);
        auto tile_rsrc = [&](const char* base, uint32_t slice, uint32_t stride, uint32_t tiles, int t) __attribute__((always_inline)) {
            const uint32_t tu = static_cast<uint32_t>(t);
            const bool inside = tu < tiles;
            const uint32_t start = tu * stride;
            return make_rsrc(inside ? base + start : base, inside ? slice - start : 0u);
        };
        // past the last tile the buffer range is empty: nothing is read
        auto issue_k = [&](int t, uint8_t* slot) __attribute__((always_inline)) {
            const auto r = tile_rsrc(kbase, kslice, kstride, ktiles, tile_at(t));
#pragma unroll
            for (int i = 0; i < KDMA; ++i) buffer_load_lds_b128(r, slot + (wave * KDMA + i) * 1024, kgo[i]);
        };
        auto issue_v = [&](int t, uint8_t* slot) __attribute__((always_inline)) {
            const auto r = tile_rsrc(vbase, vslice, vstride, vtiles, tile_at(t));
#pragma unroll
            for (int i = 0; i < VDMA; ++i) buffer_load_lds_b128(r, slot + (wave * VDMA + i) * 1024, vgo[i]);
        };

        // LDS starts as zeros so that any row the DMA does not fill holds finite values
        if (!lds_zeroed) {
            lds_zeroed = true;
            for (int i = tid; i < KTILE / 16; i += NTHREADS) {
                reinterpret_cast<u32x4*>(k_lds0)[i] = u32x4{0, 0, 0, 0};
                reinterpret_cast<u32x4*>(k_lds1)[i] = u32x4{0, 0, 0, 0};
            }
            for (int i = tid; i < VTILE / 16; i += NTHREADS) {
                reinterpret_cast<u32x4*>(v_lds0)[i] = u32x4{0, 0, 0, 0};
                reinterpret_cast<u32x4*>(v_lds1)[i] = u32x4{0, 0, 0, 0};
            }
            __syncthreads();
        }

        f32x16 oacc[CBLK];
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
        float m_run = kNegInf;   // reference max of raw scores, same in lane and lane^32
        float l_run = 0.f;       // this lane's partial row sum over its half of the keys
        float mc_run = 0.f;      // m_run * c, or 0 while m_run = -inf
        float lim = -1.f;        // largest block sum that keeps the reference: kSumLimit, or -1
                                 // while m_run = -inf (then every block takes a reference)

        // fragment addresses inside a slot (bytes)
        const int kx = kswz(col);                     // the row's chunk swizzle (same for every block)
        const int t16 = lane & 15;
        // V transposing reads: lane t of a 16-lane group points at key (k0 + t/4), channel
        // (c0 + 4*(t%4)); the group then receives, lane by lane, 16 consecutive channels of 4 keys.
        const int vkey_l = half * 4 + (t16 >> 2);                 // key offset inside a 16-key step
        const int vch_l = ((lane >> 4) & 1) * 16 + 4 * (t16 & 3); // channel offset inside a 32-block

        // K fragment of k-step kk: row (kb*32 + col), 16-byte chunk (2*kk + half) ^ kx.  The swizzle
        // only permutes chunks inside aligned groups of KSW chunks, so the address is one of
        // KSW/2 per-lane offsets plus an immediate.
        constexpr int KSW = KROWB % 256 == 0 ? 16 : 8;
        uint32_t koff[KSW / 2];
#pragma unroll
        for (int j = 0; j < KSW / 2; ++j) koff[j] = col * KROWB + ((2 * j + half) ^ kx) * 16;

        // ---- K fragment of k-step kk of the 32-key block kb of a K tile
        auto k_frag = [&](const uint8_t* kl, int kb, int kk) __attribute__((always_inline)) {
            const uint8_t* a_ptr = kl + koff[kk % (KSW / 2)] + (kk / (KSW / 2)) * KSW * 16 + kb * 32 * KROWB;
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a_ptr));
        };
        // The first KPRE fragments of a block's S are read ahead, at the end of the region before
        // the one that multiplies them, so the S MFMAs never start on an LDS read just issued.
        constexpr int KPRE = KSTEPS < 2 ? KSTEPS : 2;
        static_assert(KPRE <= KSTEPS, "prefetch at most one block's fragments");
        using KPre = bf16x8[KPRE];
        auto k_prefetch = [&](const uint8_t* kl, int kb, KPre& pre) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < KPRE; ++kk) pre[kk] = k_frag(kl, kb, kk);
        };
        // ---- S^T = K Q^T for the 32-key block kb of a K tile (one accumulator)
        auto qk_block = [&](const uint8_t* kl, int kb, f32x16& s, const KPre& pre) __attribute__((always_inline)) {
            s = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const auto a = kk < KPRE ? pre[kk] : k_frag(kl, kb, kk);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
            }
        };
        // ---- scores of keys past sk, above the diagonal or outside the window become -inf
        //      (block u of the positions: keys 32 blk_at(u) ..)
        auto need_mask = [&](int u) __attribute__((always_inline)) {
            const int key0 = blk_at(u) * 32;
            bool m = (key0 + 32 > sk) || (CAUSAL && key0 + 31 > wave_row0);
            if constexpr (EXT) {
                m = m || (p.window_left >= 0 && key0 < wave_row0 + 31 - p.window_left) ||
                    (!CAUSAL && p.window_right >= 0 && key0 + 31 > wave_row0 + p.window_right);
            }
            return m;
        };
        //      With windows or sinks compiled in, the keys the lane's row sees form one interval
        //      [key_lo, key_lo + key_range]: below sk, up to the diagonal (causal) or the right
        //      window, from the left window; a row that sees none gets [INT_MAX, INT_MAX], which
        //      no key reaches.  Score j of block u has key blk*32 + half*4 + c_j (c_j = 8*(j/4) +
        //      j%4); it is visible iff 0 <= key - key_lo <= key_range, one unsigned compare of
        //      c_j - a with a = key_lo - blk*32 - half*4 (keys, key_lo and the range all lie in
        //      [0, 2^31)): three VALU instructions per score instead of about five plus three
        //      SALU, which pays where windows put an edge in most blocks.  The plain kernels mask
        //      a block or two per wave and keep the direct test.
        [[maybe_unused]] int key_lo = 0, key_hi = sk - 1;
        if constexpr (EXT) {
            if constexpr (CAUSAL) key_hi = min(key_hi, my_row);
            if (p.window_left >= 0) key_lo = max(0, my_row - p.window_left);
            if (!CAUSAL && p.window_right >= 0 && p.window_right < key_hi - my_row) key_hi = my_row + p.window_right;
            if (key_hi < key_lo) key_lo = key_hi = INT_MAX;
        }
        [[maybe_unused]] const uint32_t key_range = static_cast<uint32_t>(key_hi) - static_cast<uint32_t>(key_lo);
        auto mask_block = [&](int u, f32x16& s) __attribute__((always_inline)) {
            if constexpr (EXT) {
                const uint32_t a = static_cast<uint32_t>(key_lo) - static_cast<uint32_t>(blk_at(u) * 32 + half * 4);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t t = static_cast<uint32_t>((j >> 2) * 8 + (j & 3)) - a;
                    if (t > key_range) s[j] = kNegInf;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = blk_at(u) * 32 + (j >> 2) * 8 + half * 4 + (j & 3);
                    if (key >= sk || (CAUSAL && key > my_row)) s[j] = kNegInf;
                }
            }
        };
        // ---- this lane's max over its 16 scores of a block
        //      (three-operand maxima: the compiler puts canonicalising moves before a maximum of
        //      scores that may come from the mask's select, and fewer of them before v_max3)
        auto lane_max = [&](const f32x16& s) __attribute__((always_inline)) {
            float a = max3(s[0], s[1], s[2]);
            float b = max3(s[8], s[9], s[10]);
            a = max3(a, s[3], s[4]);
            b = max3(b, s[11], s[12]);
            a = max3(a, s[5], s[6]);
            b = max3(b, s[13], s[14]);
            a = max3(a, s[7], s[15]);
            return __builtin_fmaxf(a, b);
        };
        // ---- the reference max: set from a block's scores (with the partner lane's half of the
        //      row), moving O and l to the new reference.  Only the first block of a row and the
        //      rare blocks that fail the check below come here.
        auto rebase = [&](const f32x16& s) __attribute__((always_inline)) {
            const float m_new = max_with_partner(lane_max(s), m_run);
            const float alpha = m_run == kNegInf ? 0.f : fast_exp2((m_run - m_new) * c);
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
            m_run = m_new;
            mc_run = m_new == kNegInf ? 0.f : m_new * c;
            lim = m_new == kNegInf ? -1.f : kSumLimit;
        };
        // ---- P^T = exp2(S^T c - m c) rounded to bf16 for score pairs [lo, hi) of a block; pair i
        //      (scores 2i, 2i+1) is word i % 4 of the B operand of 16-key P.V step i / 4
        using PWords = uint32_t[8];
        auto exp_pairs = [&](const f32x16& s, PWords& pw, auto lo_c, auto hi_c) __attribute__((always_inline)) {
#pragma unroll
            for (int i = decltype(lo_c)::value; i < decltype(hi_c)::value; ++i)
                pw[i] = pack_bf16x2(fast_exp2(fmaf(s[2 * i], c, -mc_run)), fast_exp2(fmaf(s[2 * i + 1], c, -mc_run)));
        };
        // ---- this lane's sum of the block's rounded P (the probabilities fed to P.V)
        auto block_sum = [&](const PWords& pw) __attribute__((always_inline)) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) a = add_bf16_pair(pw[i], a);
            return a;
        };
        // ---- a block u whose exponentials ran against the reference max: if any lane's sum
        //      exceeds the limit (some probability above 2^8, or a row without a reference yet),
        //      move the reference to the block's max and redo its exponentials; then add the sum
        //      to l.  The narrow heads settle a block while its scores are still live.  The wide
        //      heads settle it after its scores have died (they die as the exponentials consume
        //      them, which keeps them within 256 VGPRs): this rare path recomputes them from K in
        //      global memory, whose LDS slot may already hold a later tile, every lane loading its
        //      own fragments, bounded by the slice like the DMA, for the same MFMAs.
        auto redo = [&](const f32x16& s, PWords& pw) __attribute__((always_inline)) {
            rebase(s);
            exp_pairs(s, pw, IC<0>{}, IC<8>{});
            return block_sum(pw);
        };
        auto settle_live = [&](const f32x16& s, PWords& pw, float bs) __attribute__((always_inline)) {
            if (__any(bs > lim)) bs = redo(s, pw);
            l_run += bs;
        };
        const auto krs = make_rsrc(kbase, kslice);
        auto settle_global = [&](int u, PWords& pw, float bs) __attribute__((always_inline)) {
            if (__any(bs > lim)) {
                const int key = blk_at(u) * 32 + col;
                const uint32_t row = key < sk ? static_cast<uint32_t>(key * p.kv.ss * 2) : kOutOfRange;
                f32x16 st = f32x16{};
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) {
                    const uint32_t off = row == kOutOfRange ? kOutOfRange : row + (kk * 16 + half * 8) * 2;
                    const auto a = __builtin_bit_cast(bf16x8, buffer_load_b128(krs, off));
                    st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], st, 0, 0, 0);
                }
                if (need_mask(u)) mask_block(u, st);
                bs = redo(st, pw);
            }
            l_run += bs;
        };
        // ---- O^T += V^T P^T over the 32-key block kb of a V tile: the A operand (32 channels x
        //      16 keys) comes from two transposing reads of row-major V; keys ks*16 +
        //      {half*4 .. +3} and {8 + half*4 .. +3} match the key order of P^T's B operand
        auto pv_block = [&](const uint8_t* vl, int kb, const PWords& pw) __attribute__((always_inline)) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const auto b = __builtin_bit_cast(bf16x8, u32x4{pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]});
#pragma unroll
                for (int cb = 0; cb < CBLK; ++cb) {
                    u32x2 part[2];
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int key = kb * 32 + ks * 16 + r * 8 + vkey_l;
                        const int ch = cb * 32 + vch_l;
                        const int chunk = (ch >> 3) ^ vswz(key);
                        part[r] = lds_read_tr16_b64(vl + key * VROWB + chunk * 16 + (ch & 7) * 2);
                    }
                    const auto a = __builtin_bit_cast(bf16x8, u32x4{part[0][0], part[0][1], part[1][0], part[1][1]});
                    oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, oacc[cb], 0, 0, 0);
                }
            }
        };

        // Score pairs of block u + 1 (of 8 per lane) whose exponentials run under block u's P.V
        // MFMAs.  The wide heads run the rest, the block sum and its check under the S MFMAs of
        // block u + 2, so that the VALU work splits between the regions about as their MFMAs do;
        // the narrow heads (EARLY = 8) run all of it, sum included, under P.V and settle the block
        // right after, so that its scores die before the next S MFMAs.
        constexpr int EARLY = TileCfg<DQK, DV>::EARLY;
        constexpr bool NARROW = EARLY == 8;
        using Early = IC<EARLY>;
        // Instruction counts of the interleaved regions (per wave and 32-key block).
        constexpr int VALU_A = NARROW ? 0 : 5 * (8 - EARLY) + 8;   // FMA + exp per score, pack per pair; sum
        constexpr int PV_MFMA = 2 * CBLK;                          // two transposing V reads per MFMA
        constexpr int VALU_B = 5 * EARLY + (NARROW ? 8 : 0);
        constexpr int WAIT_VM0 = 0x0F70;                // s_waitcnt vmcnt(0)
        constexpr int VM_PROLOGUE = VDMA + KDMA;        // V_0 and K_1 may still be in flight
        constexpr int WAIT_K0 = (VM_PROLOGUE & 15) | ((VM_PROLOGUE >> 4) << 14) | 0x0F70;
        static_assert(VM_PROLOGUE < 64, "vmcnt is 6 bits");
        // region A: S of the next block (KSTEPS MFMAs, one K read each); for the wide heads also
        //           the last exponentials of the current block and its sum, which it returns
        auto region_a = [&](const uint8_t* kl, int kb, f32x16& sn, const f32x16& s, PWords& pw,
                            const KPre& pre) __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
            qk_block(kl, kb, sn, pre);
            float bs = 0.f;
            if constexpr (!NARROW) {
                exp_pairs(s, pw, Early{}, IC<8>{});
                bs = block_sum(pw);
                // keep the sum here: without a use inside the region the compiler would sink it
                asm volatile("" ::"v"(bs));
            }
            sched_region<KSTEPS, KSTEPS - KPRE, 0, 1, VALU_A, 0>(std::make_integer_sequence<int, KSTEPS>{});
            __builtin_amdgcn_sched_barrier(0);
            return bs;
        };
        // region B: P.V of the current block under the first exponentials of the next one (in
        // pw_next; for the narrow heads all of them and their sum, which it returns); with PRE,
        // it also reads the first fragments of the next region A's K block
        auto region_b = [&](const uint8_t* vl, int kb, const PWords& pw, const f32x16& sn, PWords& pw_next,
                            auto vmem_c, auto pre_c, const uint8_t* kl_next, int kb_next,
                            KPre& pre) __attribute__((always_inline)) {
            constexpr int NPRE = decltype(pre_c)::value ? KPRE : 0;
            pv_block(vl, kb, pw);
            exp_pairs(sn, pw_next, IC<0>{}, Early{});
            float bs = 0.f;
            if constexpr (NARROW) {
                bs = block_sum(pw_next);
                asm volatile("" ::"v"(bs));
            } else {
                // keep the exponentials here: without a use inside the region the compiler would
                // sink them to the region that consumes them
#pragma unroll
                for (int i = 0; i < EARLY; ++i) asm volatile("" ::"v"(pw_next[i]));
            }
            if constexpr (NPRE > 0) k_prefetch(kl_next, kb_next, pre);
            sched_region<PV_MFMA, 2 * PV_MFMA + NPRE, 2 * CBLK, 2, VALU_B, decltype(vmem_c)::value>(
                std::make_integer_sequence<int, PV_MFMA>{});
            __builtin_amdgcn_sched_barrier(0);
            return bs;
        };

        // ---- main loop over 64-key tiles, software-pipelined over their 32-key blocks (block u's
        //      probabilities are finished and checked in the region A that runs the S MFMAs of
        //      block u+1 (wide heads) or in the region B before it (narrow heads); block u's P.V
        //      runs in the region B after it).  Tile t's K sits in k slot t%2 and its V in v slot
        //      t%2; even blocks keep their scores in s0 and probabilities in p0, odd ones in
        //      s1 / p1.  The barrier of iteration t (after the S MFMAs of its second block)
        //      guarantees that every wave's part of V_t and K_{t+1} has landed and that no wave
        //      still reads K_t or V_{t-1}: their slots then take K_{t+2} and V_{t+1}.
        using NoVmem = IC<0>;
        using DmaVmem = IC<KDMA + VDMA>;
        using Pre = std::true_type;
        using NoPre = std::false_type;
        auto iteration = [&](int t, auto par_c, f32x16& s0, f32x16& s1, PWords& p0, PWords& p1, KPre& pre)
                             __attribute__((always_inline)) {
            using Cur = IC<decltype(par_c)::value>;
            using Nxt = IC<decltype(par_c)::value ^ 1>;
            // block 2t (s0, p0) with the S of block 2t+1 (into s1)
            float bs = region_a(k_slot(Cur{}), 1, s1, s0, p0, pre);
            if (need_mask(2 * t + 1)) mask_block(2 * t + 1, s1);
            if constexpr (!NARROW) settle_global(2 * t, p0, bs);
            __builtin_amdgcn_s_waitcnt(WAIT_VM0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            issue_k(t + 2, k_slot(Cur{}));
            issue_v(t + 1, v_slot(Nxt{}));
            bs = region_b(v_slot(Cur{}), 0, p0, s1, p1, DmaVmem{}, Pre{}, k_slot(Nxt{}), 0, pre);
            if constexpr (NARROW) settle_live(s1, p1, bs);
            // block 2t+1 (s1, p1) with the S of block 2t+2, the first block of the next tile (into s0)
            bs = region_a(k_slot(Nxt{}), 0, s0, s1, p1, pre);
            if (need_mask(2 * t + 2)) mask_block(2 * t + 2, s0);
            if constexpr (!NARROW) settle_global(2 * t + 1, p1, bs);
            __builtin_amdgcn_sched_barrier(0);
            // the next region A (an iteration or the last tile) starts on block 1 of K_{t+1}
            bs = region_b(v_slot(Cur{}), 1, p1, s0, p0, NoVmem{}, Pre{}, k_slot(Nxt{}), 1, pre);
            if constexpr (NARROW) settle_live(s0, p0, bs);
        };
        // the last tile: its two blocks, nothing further to load
        auto last = [&](int t, auto par_c, const f32x16& s0, f32x16& s1, PWords& p0, PWords& p1, KPre& pre)
                        __attribute__((always_inline)) {
            using Cur = IC<decltype(par_c)::value>;
            float bs = region_a(k_slot(Cur{}), 1, s1, s0, p0, pre);
            if (need_mask(2 * t + 1)) mask_block(2 * t + 1, s1);
            if constexpr (!NARROW) settle_global(2 * t, p0, bs);
            __builtin_amdgcn_s_waitcnt(WAIT_VM0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            bs = region_b(v_slot(Cur{}), 0, p0, s1, p1, NoVmem{}, NoPre{}, nullptr, 0, pre);
            if constexpr (NARROW) {
                settle_live(s1, p1, bs);
            } else {
                exp_pairs(s1, p1, Early{}, IC<8>{});
                settle_live(s1, p1, block_sum(p1));
            }
            pv_block(v_slot(Cur{}), 1, p1);
        };

        if (ntiles > t0) {
            using Zero = IC<0>;
            using One = IC<1>;
            issue_k(t0, k_slot(Zero{}));
            issue_v(t0, v_slot(Zero{}));
            issue_k(t0 + 1, k_slot(One{}));
            // softmax(c * s) with c < 0 equals softmax(|c| * (-s)): negate Q (exact) and use |c|.
            // The flip needs Q's data, so it stays behind the DMA requests: the K/V round trip
            // then overlaps Q's instead of starting after it.
            __builtin_amdgcn_sched_barrier(0);
            if (p.scale_log2 < 0.f) {
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk)
                    qf[kk] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[kk]) ^ 0x80008000u);
            }
            __builtin_amdgcn_s_waitcnt(WAIT_K0);   // this wave's part of K_t0 has landed
            __syncthreads();
            f32x16 s0, s1;
            PWords p0, p1;
            KPre pre;
            if constexpr (!CAN_REV) {
                k_prefetch(k_slot(Zero{}), 0, pre);
                qk_block(k_slot(Zero{}), 0, s0, pre);
                if (need_mask(2 * t0)) mask_block(2 * t0, s0);
                rebase(s0);                           // the row's first reference max
                exp_pairs(s0, p0, IC<0>{}, Early{});
                if constexpr (NARROW) l_run = block_sum(p0);
                k_prefetch(k_slot(Zero{}), 1, pre);   // the first region A starts on block 1 of K_t0
                // Tiles up to `need` hold a key that some row of this wave sees; past them (the
                // diagonal tiles of the rows above, or right of a window) the wave only keeps the
                // ring's waits, barriers and its share of the DMA.  Wave-uniform.
                int need = ntiles;
                if constexpr (CAUSAL) need = min(ntiles, (wave_row0 + 31) / BN + 1);
                if constexpr (EXT && !CAUSAL) {
                    if (p.window_right >= 0) need = min(ntiles, (wave_row0 + 31 + p.window_right) / BN + 1);
                }
                const int e = min(need, ntiles - 1);   // tiles run through iteration()
                int t = t0;
                for (; t + 2 <= e; t += 2) {
                    iteration(t, Zero{}, s0, s1, p0, p1, pre);
                    iteration(t + 1, One{}, s0, s1, p0, p1, pre);
                }
                const bool odd = t < e;
                if (odd) iteration(t++, Zero{}, s0, s1, p0, p1, pre);
                if (need == ntiles) {
                    if (odd) last(t, One{}, s0, s1, p0, p1, pre);
                    else last(t, Zero{}, s0, s1, p0, p1, pre);
                } else {
                    // tile t has parity (t - t0) & 1; the last tile issues no further DMA
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
            } else {
                // Causal, t0 = 0: every row sees key 0, so every wave runs to the last position.
                // Upward, a wave stops computing after its diagonal tile and drains the rest;
                // downward, it drains the tiles above its rows first and starts on block 0 of its
                // diagonal tile, which holds a key that every row of the wave sees.  Either way
                // each wave keeps one barrier per position.  Wave-uniform.
                //
                // a position the wave does not compute keeps the ring's wait, barrier and its share
                // of the DMA; position t has parity (t - t0) & 1
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
                // the wave's first block (block 0 of the tile at position u, ring slot par_c): its
                // scores set the reference max
                auto first_block = [&](int u, auto par_c) __attribute__((always_inline)) {
                    using Cur = IC<decltype(par_c)::value>;
                    k_prefetch(k_slot(Cur{}), 0, pre);
                    qk_block(k_slot(Cur{}), 0, s0, pre);
                    if (need_mask(2 * u)) mask_block(2 * u, s0);
                    rebase(s0);
                    exp_pairs(s0, p0, IC<0>{}, Early{});
                    if constexpr (NARROW) l_run = block_sum(p0);
                    k_prefetch(k_slot(Cur{}), 1, pre);   // the first region A starts on block 1
                };
                const int need = min(ntiles, (wave_row0 + 31) / BN + 1);
                int t = t0;
                for (const int first = rev ? t0 + ntiles - need : t0; t < first; ++t) {
                    if ((t - t0) & 1) drain(t, One{});
                    else drain(t, Zero{});
                }
                const int stop = rev ? ntiles : need;   // positions [t, stop) are computed
                const int e = min(stop, ntiles - 1);    // through iteration()
                bool odd = (t - t0) & 1;
                if (!odd) {
                    first_block(t, Zero{});
                } else {
                    first_block(t, One{});
                    if (t < e) {
                        iteration(t++, One{}, s0, s1, p0, p1, pre);
                        odd = false;
                    }
                }
                for (; t + 2 <= e; t += 2) {
                    iteration(t, Zero{}, s0, s1, p0, p1, pre);
                    iteration(t + 1, One{}, s0, s1, p0, p1, pre);
                }
                if (!odd && t < e) {
                    iteration(t++, Zero{}, s0, s1, p0, p1, pre);
                    odd = true;
                }
                if (stop == ntiles) {
                    if (odd) last(t, One{}, s0, s1, p0, p1, pre);
                    else last(t, Zero{}, s0, s1, p0, p1, pre);
                } else {
                    bool par = odd;
                    for (; t < ntiles; ++t) {
                        if (par) drain(t, One{});
                        else drain(t, Zero{});
                        par = !par;
                    }
                }
            }
        }

        // ---- epilogue: normalise, store O (bf16) and LSE
        float l_tot = l_run + swap_halves(l_run);
        float m_log2 = m_run * c;   // the reference max in base-2 units (c > 0 keeps -inf)
        float o_scale = 1.f;
        if constexpr (SPLIT) {
            // this key range's state goes to the workspace and the merge kernel finishes the row:
            // O unnormalised, in accumulator order (the merge reads it back lane for lane), and
            // per lane the base-2 reference max and the row sum
            const int64_t slot = ((static_cast<int64_t>(item) * p.n_split + split) * (CAUSAL ? 2 : 1) + which) * NWAVES + wave;
            float* po = p.split_o + slot * (CBLK * 16 * 64);
#pragma unroll
            for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 w = {oacc[cb][4 * q4], oacc[cb][4 * q4 + 1], oacc[cb][4 * q4 + 2], oacc[cb][4 * q4 + 3]};
                    *reinterpret_cast<f32x4*>(po + ((cb * 4 + q4) * 64 + lane) * 4) = w;
                }
            }
            reinterpret_cast<f32x2*>(p.split_ml)[slot * 64 + lane] = f32x2{m_log2, l_tot};
            if constexpr (PAIRED) goto item_done;
            else return;
        }
        if constexpr (EXT) {
            // the head's sink logit joins the normaliser: rebase both terms on their larger
            // exponent so that neither overflows
            if (p.sinks != nullptr) {
                const float s2 = p.sinks[h] * kLog2e;
                const float top = fmaxf(m_log2, s2);
                if (top != kNegInf) {
                    o_scale = m_log2 == kNegInf ? 0.f : fast_exp2(m_log2 - top);
                    l_tot = l_tot * o_scale + fast_exp2(s2 - top);
                    m_log2 = top;
                }
            }
        }
        const float inv = l_tot > 0.f ? o_scale / l_tot : 0.f;
        if (my_row < sq) {
            uint16_t* orow = static_cast<uint16_t*>(p.o) + (orow0 + h * p.ov.sh + my_row * p.ov.ss);
            store_o_row<CBLK>(orow, oacc, inv, half);
            if (p.lse != nullptr && half == 0) {
                const float lse = l_tot > 0.f ? (m_log2 + __log2f(l_tot)) * kLn2 : kNegInf;
                p.lse[lse0 + my_row] = lse;
            }
        }
    }
item_done: __attribute__((unused));
    if constexpr (PAIRED) {
        // the pair's light block: the slots are rewritten only after every wave is done
        bool more = mblk != mrev;
        if constexpr (SPLIT) more = which == 0 && pair_b > pair_la && pair_lb > 0;
        if (more) {
            mblk = mrev;
            if constexpr (SPLIT) {
                which = 1;
                seg0 = 0;
                seg1 = pair_b - pair_la;
            }
            __syncthreads();
            goto next_item;
        }
    }
}

// The key-range split's second kernel: one workgroup per (query block, 32-channel block of O),
// laid out like the attention kernel (one wave per 32 rows, the same lanes), merges the partial
// states of the ranges that cover the block, in ascending order of range.  The softmax over the
// union of the ranges is
//   O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i,   M = max_i m_i   (base-2 units),
// and LSE = (M + log2 of the denominator) ln 2, so the result does not depend on timing.  (Every
// channel block's workgroup recomputes the row's weights from the same values, in the same
// order; the first one writes the LSE.)  Causal grids split pairs of blocks (n-1-j, j): ranges
// [r L / n_split, (r + 1) L / n_split) of the pair's L = LA + LB tiles; block n-1-j takes the
// ranges that start before LA, block j those that end after it.
template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__((TileCfg<DQK, DV>::BM * 2)) void attn_split_merge(const AttnParams p) {
    constexpr int BM = TileCfg<DQK, DV>::BM;
    constexpr int BN = TileCfg<DQK, DV>::BN;
    constexpr int NWAVES = BM / 32;
    constexpr int CBLK = DV / 32;
    constexpr int OWAVE = CBLK * 16 * 64;
    const int cb = blockIdx.x % CBLK;
    const int unit = blockIdx.x / CBLK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    int item, which = 0, mblk, bh, la = 0, len = 0;
    if constexpr (CAUSAL) {
        item = unit >> 1;
        which = unit & 1;
        const int per_head = (p.n_mblocks + 1) / 2;
        const int mrev = item % per_head;
        const int ma = p.n_mblocks - 1 - mrev;
        if (which == 1 && ma == mrev) return;   // an odd count's middle block is one item
        bh = item / per_head;
        mblk = which ? mrev : ma;
        la = split_causal_tiles<BM, BN>(ma, p.sk);
        len = la + (ma != mrev ? split_causal_tiles<BM, BN>(mrev, p.sk) : 0);
    } else {
        item = unit;
        mblk = item % p.n_mblocks;
        bh = item / p.n_mblocks;
    }
    auto covers = [&](int r) __attribute__((always_inline)) {
        if constexpr (!CAUSAL) return true;
        return which == 0 ? r * len / p.n_split < la : (r + 1) * len / p.n_split > la;
    };
    const int h = bh % p.hq;
    const int bb = bh / p.hq;
    const int my_row = mblk * BM + wave * 32 + col;
    auto slot = [&](int r) __attribute__((always_inline)) {
        return ((static_cast<int64_t>(item) * p.n_split + r) * (CAUSAL ? 2 : 1) + which) * NWAVES + wave;
    };
    const f32x2* pml = reinterpret_cast<const f32x2*>(p.split_ml) + lane;
    float mmax = kNegInf;
    for (int r = 0; r < p.n_split; ++r)
        if (covers(r)) mmax = fmaxf(mmax, pml[slot(r) * 64][0]);
    f32x16 acc[1] = {f32x16{}};
    float lsum = 0.f;
    for (int r = 0; r < p.n_split; ++r) {
        if (!covers(r)) continue;
        const f32x2 ml = pml[slot(r) * 64];
        const float w = ml[0] == kNegInf ? 0.f : fast_exp2(ml[0] - mmax);
        lsum = fmaf(w, ml[1], lsum);
        const float* po = p.split_o + slot(r) * OWAVE;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(po + ((cb * 4 + q4) * 64 + lane) * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[0][4 * q4 + j] = fmaf(w, x[j], acc[0][4 * q4 + j]);
        }
    }
    if (my_row < p.sq) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        uint16_t* orow = static_cast<uint16_t*>(p.o) +
                         (static_cast<int64_t>(bb) * p.ov.sb + h * p.ov.sh + my_row * p.ov.ss) + cb * 32;
        store_o_row<1>(orow, acc, inv, half);
        if (cb == 0 && p.lse != nullptr && half == 0) {
            const float lse = lsum > 0.f ? (mmax + __log2f(lsum)) * kLn2 : kNegInf;
            p.lse[(static_cast<int64_t>(bb) * p.hq + h) * p.sq + my_row] = lse;
        }
    }
}

template <int DQK, int DV, bool CAUSAL, bool VARLEN>
hipError_t launch(AttnParams p, hipStream_t stream) {
    constexpr int BM = TileCfg<DQK, DV>::BM;
    p.n_mblocks = (p.sq + BM - 1) / BM;
    const int64_t blocks = static_cast<int64_t>(p.b) * p.hq * p.n_mblocks;
    if (blocks == 0) return hipSuccess;
    // Pair causal query blocks, so that every workgroup does the same work and the in-order
    // dispatch never waits behind a long one (measured: -5 to -10% on grids of 2-8 rounds of
    // resident workgroups, -1.7% on the 16-round MLA grid, -2.6% on d128 8192^2 hq128).  Packed
    // sequences pair only on grids of at most 8 rounds: their workgroups are dealt to the XCDs
    // by (sequence, kv head), and pairing the 32-sequence workload's 8192-row grid cost +11%.
    const bool ext = p.window_left >= 0 || (!CAUSAL && p.window_right >= 0) || p.sinks != nullptr;
    if (p.n_split > 1) {
        if constexpr (VARLEN) {
            return hipErrorInvalidValue;
        } else {
            if (ext || p.split_ml == nullptr || p.split_o == nullptr) return hipErrorInvalidValue;
            // units: query blocks, or causal pairs (n-1-j, j); the merge has one workgroup per
            // (block, 32-channel block), two blocks per pair
            const int64_t units = CAUSAL ? static_cast<int64_t>(p.b) * p.hq * ((p.n_mblocks + 1) / 2) : blocks;
            const int64_t nwg = units * p.n_split;
            const int64_t nmerge = units * (CAUSAL ? 2 : 1) * (DV / 32);
            if (nwg > INT32_MAX || nmerge > INT32_MAX) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, CAUSAL, false, CAUSAL, false, true>),
                               dim3(static_cast<unsigned>(nwg)), dim3(BM * 2), 0, stream, p);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((attn_split_merge<DQK, DV, CAUSAL>), dim3(static_cast<unsigned>(nmerge)), dim3(BM * 2), 0,
                               stream, p);
            return hipGetLastError();
        }
    }
    if (ext) {
        if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        // sinks (and right windows) under GQA: two query heads per workgroup as below (d64,
        // d128).  Not with a left window: its blocks see few keys each and are bound by the
        // latency of their first loads, which more, smaller workgroups per CU hide better (the
        // 128-key window layer of the GPT-OSS shape: 71.0 -> 75.2 us packed; its full layer
        // with sinks: 621 -> 600 us)
        if constexpr ((DQK == 64 || DQK == 128) && DQK == DV && MHA_HEADS_PER_WG > 1) {
            constexpr int H = MHA_HEADS_PER_WG;
            if (p.group % H == 0 && p.window_left < 0) {
                const auto kernel = attn_fwd_bf16_kernel<DQK, DV, CAUSAL, VARLEN, false, true, false, H>;
                int groups = 0;
                const hipError_t e = resident_groups(reinterpret_cast<const void*>(kernel), BM * 2 * H, &groups);
                if (e != hipSuccess) return e;
                const int64_t nwg = static_cast<int64_t>(p.b) * (p.hq / H) * p.n_mblocks;
                if (nwg >= groups) {
                    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(nwg)), dim3(BM * 2 * H), 0, stream, p);
                    return hipGetLastError();
                }
            }
        }
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, CAUSAL, VARLEN, false, true, false>),
                           dim3(static_cast<unsigned>(blocks)), dim3(BM * 2), 0, stream, p);
        return hipGetLastError();
    }
    bool paired = CAUSAL && p.n_mblocks > 1;
    // d128 under GQA: two query heads per workgroup, when the grid still fills the device (packed
    // sequences pair blocks by the same rule as below)
    if constexpr (DQK == 128 && DV == 128 && MHA_HEADS_PER_WG > 1) {
        constexpr int H = MHA_HEADS_PER_WG;
        if (p.group % H == 0) {
            const auto paired_kernel = attn_fwd_bf16_kernel<DQK, DV, CAUSAL, VARLEN, CAUSAL, false, false, H>;
            const auto plain_kernel = attn_fwd_bf16_kernel<DQK, DV, CAUSAL, VARLEN, false, false, false, H>;
            int groups = 0;
            const hipError_t e = resident_groups(reinterpret_cast<const void*>(plain_kernel), BM * 2 * H, &groups);
            if (e != hipSuccess) return e;
            const int64_t blocks_h = static_cast<int64_t>(p.b) * (p.hq / H) * p.n_mblocks;
            bool paired_h = paired;
            if (paired_h && VARLEN) paired_h = blocks_h <= 8 * static_cast<int64_t>(groups);
            const int64_t nwg = paired_h ? static_cast<int64_t>(p.b) * (p.hq / H) * ((p.n_mblocks + 1) / 2) : blocks_h;
            if (nwg >= groups) {
                if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
                hipLaunchKernelGGL(paired_h ? paired_kernel : plain_kernel, dim3(static_cast<unsigned>(nwg)), dim3(BM * 2 * H),
                                   0, stream, p);
                return hipGetLastError();
            }
        }
    }
    if (paired && VARLEN) {
        int groups = 0;
        const auto kernel = attn_fwd_bf16_kernel<DQK, DV, CAUSAL, VARLEN, CAUSAL, false, false>;
        const hipError_t e = resident_groups(reinterpret_cast<const void*>(kernel), BM * 2, &groups);
        if (e != hipSuccess) return e;
        paired = blocks <= 8 * static_cast<int64_t>(groups);
    }
    const int64_t nwg = paired ? static_cast<int64_t>(p.b) * p.hq * ((p.n_mblocks + 1) / 2) : blocks;
    if (nwg > INT32_MAX) return hipErrorInvalidConfiguration;
    if (paired) {
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, CAUSAL, VARLEN, CAUSAL, false, false>), dim3(static_cast<unsigned>(nwg)),
                           dim3(BM * 2), 0, stream, p);
    } else {
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, CAUSAL, VARLEN, false, false, false>), dim3(static_cast<unsigned>(nwg)),
                           dim3(BM * 2), 0, stream, p);
    }
    return hipGetLastError();
}

template <bool VARLEN>
hipError_t launch_dims(const AttnParams& p, int d_qk, int d_v, bool causal, hipStream_t stream) {
    if (d_qk == 32 && d_v == 32)
        return causal ? launch<32, 32, true, VARLEN>(p, stream) : launch<32, 32, false, VARLEN>(p, stream);
    if (d_qk == 64 && d_v == 64)
        return causal ? launch<64, 64, true, VARLEN>(p, stream) : launch<64, 64, false, VARLEN>(p, stream);
    if (d_qk == 128 && d_v == 128)
        return causal ? launch<128, 128, true, VARLEN>(p, stream) : launch<128, 128, false, VARLEN>(p, stream);
    if (d_qk == 192 && d_v == 128)
        return causal ? launch<192, 128, true, VARLEN>(p, stream) : launch<192, 128, false, VARLEN>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnParams& p, int d_qk, int d_v, bool causal, hipStream_t stream) {
    return p.cu_q != nullptr ? launch_dims<true>(p, d_qk, d_v, causal, stream)
                             : launch_dims<false>(p, d_qk, d_v, causal, stream);
}

namespace {

// rows per workgroup and the split kernel of a head-dim pair (nullptr: not built)
template <int DQK, int DV>
const void* split_kernel(bool causal, int* bm) {
    *bm = TileCfg<DQK, DV>::BM;
    return causal ? reinterpret_cast<const void*>(attn_fwd_bf16_kernel<DQK, DV, true, false, true, false, true>)
                  : reinterpret_cast<const void*>(attn_fwd_bf16_kernel<DQK, DV, false, false, false, false, true>);
}

const void* split_kernel_for(int d_qk, int d_v, bool causal, int* bm) {
    if (d_qk == 32 && d_v == 32) return split_kernel<32, 32>(causal, bm);
    if (d_qk == 64 && d_v == 64) return split_kernel<64, 64>(causal, bm);
    if (d_qk == 128 && d_v == 128) return split_kernel<128, 128>(causal, bm);
    if (d_qk == 192 && d_v == 128) return split_kernel<192, 128>(causal, bm);
    return nullptr;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kSplitBN = 64;   // key tile of every TileCfg

// Key tiles per range: non-causal, the ceil(sk / 64) tiles of every block (`shortest` as
// `longest`); causal, the pair lengths LA + LB, the shortest and the longest.
void split_lengths(int n_mblocks, int bm, int sk, bool causal, int* shortest, int* longest) {
    if (!causal) {
        *shortest = *longest = (sk + kSplitBN - 1) / kSplitBN;
        return;
    }
    auto tiles = [&](int m) {
        const int64_t keys = std::min<int64_t>(static_cast<int64_t>(m + 1) * bm, sk);
        return static_cast<int>((keys + kSplitBN - 1) / kSplitBN);
    };
    int lo = INT32_MAX, hi = 0;
    for (int j = 0; j < (n_mblocks + 1) / 2; ++j) {
        const int ma = n_mblocks - 1 - j;
        const int len = tiles(ma) + (ma != j ? tiles(j) : 0);
        lo = std::min(lo, len);
        hi = std::max(hi, len);
    }
    *shortest = n_mblocks > 0 ? lo : 0;
    *longest = hi;
}

}  // namespace

size_t attn_bf16_split_layout(int b, int hq, int sq, int d_qk, int d_v, int n_split, size_t offsets[2]) {
    int bm = 0;
    if (split_kernel_for(d_qk, d_v, false, &bm) == nullptr || b < 0 || hq < 0 || sq < 0 || n_split < 1) return 0;
    // two block slots per pair of blocks: the causal pairs (n-1-j, j), and at least the blocks
    const size_t nmb = (static_cast<size_t>(sq) + bm - 1) / bm;
    const size_t slots = static_cast<size_t>(b) * hq * 2 * ((nmb + 1) / 2);
    const size_t waves = static_cast<size_t>(bm / 32);
    offsets[0] = 0;
    offsets[1] = round256(slots * n_split * waves * 64 * 2 * sizeof(float));
    return offsets[1] + round256(slots * n_split * static_cast<size_t>(bm) * d_v * sizeof(float));
}

int attn_bf16_split_max(int sq, int sk, int d_qk, int d_v, bool causal) {
    int bm = 0;
    if (split_kernel_for(d_qk, d_v, causal, &bm) == nullptr || sq <= 0 || sk <= 0) return 0;
    int shortest = 0, longest = 0;
    split_lengths((sq + bm - 1) / bm, bm, sk, causal, &shortest, &longest);
    return shortest;
}

hipError_t attn_bf16_split_plan(int b, int hq, int sq, int sk, int d_qk, int d_v, bool causal, int* n_split) {
    *n_split = 1;
    int bm = 0;
    const void* kernel = split_kernel_for(d_qk, d_v, causal, &bm);
    if (kernel == nullptr || b <= 0 || hq <= 0 || sq <= 0 || sk <= 0) return hipSuccess;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cus <= 0) return hipSuccess;
    // A model of the time in microseconds, calibrated on MI355X (d128, 8192^2, measured):
    //  * k workgroups on a CU share its throughput, ~4.5 TFLOP/s per CU when every SIMD holds two
    //    waves; one 4-wave workgroup alone (one wave per SIMD) runs at 0.87 of that;
    //  * a split workgroup adds about one key tile of prologue and partial stores;
    //  * the merge reads the fp32 partials at ~5 TB/s, plus ~3 us for its launch.
    // It reproduces the measured choices: the GQA 5:1 non-causal shape (320 blocks) gains 12-13%
    // at three ranges; the GQA 8:1 shapes, causal (256 pairs, one per CU) or not, lose at every
    // split.  The split with the least predicted time is taken (the fewest ranges within 3% of
    // it) if it beats the unsplit grid by 10%, and only with ranges of keys x (d_qk + d_v) >= 2^18,
    // 1024 keys at d128, below which fixed costs dominate (a d32 2048^2 shape loses at every split).
    // Causal grids split pairs of blocks (n-1-j, j), whose tile counts L = LA + LB are close to equal.
    const int nmb = (sq + bm - 1) / bm;
    const int64_t units = static_cast<int64_t>(b) * hq * (causal ? (nmb + 1) / 2 : nmb);
    int shortest = 0, nt = 0;
    split_lengths(nmb, bm, sk, causal, &shortest, &nt);
    const double t_tile = static_cast<double>(bm) * kSplitBN * (d_qk + d_v) * 2.0 / 4.5e12 * 1e6;
    const int waves = bm / 32;
    auto cost = [&](int s) {
        const int64_t k = (units * s + cus - 1) / cus;
        const double tiles = static_cast<double>(nt) / s + (s > 1 ? 1.0 : 0.0);
        double t = static_cast<double>(k) * tiles * t_tile / (k * waves < 8 ? 0.87 : 1.0);
        if (s > 1) {
            const double slots = causal ? units * (s + 1.0) : static_cast<double>(units) * s;
            t += slots * bm * d_v * 4.0 / 5.0e12 * 1e6 + 3.0;
        }
        return t;
    };
    double costs[9] = {0};
    int top = 1;
    for (int s = 2; s <= 8 && s <= shortest && units * s <= INT32_MAX &&
                    static_cast<int64_t>(nt / s) * kSplitBN * (d_qk + d_v) >= (int64_t(1) << 18);
         ++s)
        top = s;
    double best = cost(1);
    for (int s = 1; s <= top; ++s) {
        costs[s] = cost(s);
        best = std::min(best, costs[s]);
    }
    if (best >= 0.9 * costs[1]) return hipSuccess;
    for (int s = 2; s <= top; ++s) {
        if (costs[s] <= 1.03 * best) {
            *n_split = s;
            break;
        }
    }
    return hipSuccess;
}

}  // namespace mha
