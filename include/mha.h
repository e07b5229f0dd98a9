/*
 * mha.h - C ABI of the MI355X (gfx950) fused attention forward library (libmha.so).
 *
 * Operations, each enqueued on the caller's HIP stream:
 *
 *   mha_fwd_bf16   fused attention forward, bf16 in / bf16 out, fp32 accumulate
 *   mha_fwd_bf16_varlen  the same over packed sequences (cumulative offsets)
 *   mha_fwd_bf16_window_sink  the same with a sliding window and attention sinks
 *   mha_fwd_bf16_varlen_window_sink  both
 *   k_smooth_mean  per-(batch, kv head) K mean behind a gate (two kernels, one call)
 *   mha_fwd_fp8    K-smoothed FP8 (E4M3) block-quantised attention forward
 *   mha_fwd_mxfp8  the same with MXFP8 (E8M0 exponent per 32 channels) quantisation
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Tensors are BSHD views: element (b, s, h, c) lives at
 *       base + b*stride.b + s*stride.s + h*stride.h + c        (element units)
 *   i.e. the channel dimension is contiguous (stride 1) and the other three
 *   strides are free (head-sliced or packed-QKV views are fine).  Strides are
 *   non-negative.
 *
 *   All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   allocates no device memory and keeps no state between calls other than a
 *   host-side cache of each kernel's occupancy per device (used to size grids);
 *   where a call needs scratch space the caller passes a workspace whose size
 *   is given by the matching *_workspace_bytes() query.
 *
 *   `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Calls return after enqueueing; nothing synchronises.  Kernel faults
 *   therefore surface at a later synchronisation.
 *
 *   Every argument is validated on the host before anything is launched; a
 *   refusal returns a non-zero status, launches nothing, and leaves a message
 *   naming the offending argument in mha_last_error() (thread-local).
 *
 *   Head mapping (GQA): query head h reads kv head h / (hq / hk).
 *   Causal mask: top-left aligned, key j is visible to query i iff j <= i.
 *   LSE: natural-log log-sum-exp of the scaled, masked scores of each row,
 *   fp32, contiguous [b, hq, sq]; a row with no visible key (sk == 0) gets
 *   O = 0 and LSE = -inf.
 *
 *   Results are deterministic: the same inputs give bitwise-identical outputs
 *   (no atomics, fixed reduction orders).
 */
#ifndef MHA_H_
#define MHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MHA_OK = 0,
    MHA_ERR_NULL = 1,         /* a required pointer is NULL                          */
    MHA_ERR_SHAPE = 2,        /* a size is negative, or hq is not a multiple of hk   */
    MHA_ERR_UNSUPPORTED = 3,  /* head dims / dtype combination not built             */
    MHA_ERR_LAYOUT = 4,       /* misaligned pointer or stride, negative stride       */
    MHA_ERR_OVERFLOW = 5,     /* an in-kernel 32-bit offset or extent would overflow  */
    MHA_ERR_WORKSPACE = 6,    /* workspace missing, misaligned or too small          */
    MHA_ERR_HIP = 7,          /* the HIP runtime reported an error at launch         */
    MHA_ERR_VALUE = 8         /* a scalar argument is out of range (non-finite scale) */
} mha_status;

/* Element strides of a BSHD view; the channel stride is 1 by contract. */
typedef struct {
    int64_t b;
    int64_t s;
    int64_t h;
} mha_strides;

/*
 * mha_fwd_bf16 - fused attention forward pass in bf16.
 *
 * Computes O = softmax(softmax_scale * Q K^T + causal mask) V and the per-row
 * LSE: the MHA forward pass of "Tune MHA config & small-head pipeline
 * pathology" (Motivation; Test Plan: causal/non-causal, GQA 48:8, head_dim 64,
 * and the dqk=192 / dv=128 MLA-prefill "PE" bucket).
 *
 *   q    [b, sq, hq, d_qk] bf16      k [b, sk, hk, d_qk] bf16
 *   v    [b, sk, hk, d_v]  bf16      o [b, sq, hq, d_v]  bf16 (written)
 *   lse  [b, hq, sq] fp32 contiguous (written), or NULL to skip it
 *   (d_qk, d_v) in {(32, 32), (64, 64), (128, 128), (192, 128)} (32: the small-head
 *   "vd32" shapes of the same page's Test Result table)
 *   b, sq, sk >= 0; hq, hk >= 1; hq % hk == 0.  b == 0 or sq == 0 is a no-op.
 *   softmax_scale: any finite value (usually 1/sqrt(d_qk)).
 *   causal: 0 or 1.
 *
 * Layout requirements: q, k, v, o 16-byte aligned and every stride a
 * multiple of 8 elements (16-byte rows); key rows of k and v must not overlap
 * (stride.s >= d when sk > 1); lse 4-byte aligned.  Each (b, head)
 * slice of q/k/v/o must span < 2^31 bytes.  Accumulation is fp32; O is
 * rounded to bf16 once at the end.
 */
mha_status mha_fwd_bf16(const void* q, mha_strides q_stride,
                        const void* k, mha_strides k_stride,
                        const void* v, mha_strides v_stride,
                        void* o, mha_strides o_stride,
                        float* lse,
                        int b, int hq, int hk, int sq, int sk, int d_qk, int d_v,
                        float softmax_scale, int causal, void* stream);

/*
 * mha_fwd_bf16_split - mha_fwd_bf16 with each query block's keys divided among
 * n_split workgroups, for grids of few query blocks that would leave compute
 * units idle: the per-rank shapes of "Tune MHA config & small-head pipeline
 * pathology" (The 8 remaining regressions: d128 8192^2 at TP8, hq8/hk1 and
 * hq5/hk1), whose 320-512 query blocks of 128 rows are one round of the
 * device or less.  Non-causal: each workgroup runs keys [t0*64, t1*64) for its
 * range of the ceil(sk/64) key tiles (the ranges differ by at most one tile).
 * Causal: the blocks are paired (n-1-j, j) as in the unsplit call, and the
 * L = LA + LB key tiles of a pair (block n-1-j's, then block j's) are divided
 * the same way, so a range may end in one block and go on in the other.  Each
 * workgroup leaves an fp32 state per block it touches in the workspace; a
 * second kernel on the same stream merges, per block, the ranges that cover it
 * in ascending order through the softmax identity over a union of key sets,
 *   O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i,
 * which is the LSE merge of the same page's outputs (O, LSE).  The result is
 * deterministic but not bitwise the unsplit one: the probabilities are rounded
 * to bf16 against each range's own reference max and the sums run in another
 * order (both within the unsplit call's error bounds).
 *
 *   n_split  1 (exactly mha_fwd_bf16; ws ignored) to 16, and at most the key
 *            tiles of 64 of the shortest block (non-causal: ceil(sk/64)) or
 *            pair of blocks (causal), else MHA_ERR_VALUE
 *   ws       device workspace of at least
 *            mha_fwd_bf16_split_workspace_bytes(b, hq, sq, d_qk, d_v, n_split)
 *            bytes, 256-byte aligned (else MHA_ERR_WORKSPACE).  Its contents
 *            need no initialisation and are scratch after the call; calls that
 *            overlap in time (another stream) need separate workspaces.
 * Everything else (shapes, layouts, errors) as mha_fwd_bf16.  Two kernels run
 * on `stream`: the attention kernel, then the merge.
 */
mha_status mha_fwd_bf16_split(const void* q, mha_strides q_stride,
                              const void* k, mha_strides k_stride,
                              const void* v, mha_strides v_stride,
                              void* o, mha_strides o_stride,
                              float* lse,
                              int b, int hq, int hk, int sq, int sk, int d_qk, int d_v,
                              float softmax_scale, int causal,
                              int n_split, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace mha_fwd_bf16_split needs for n_split ranges: for each
 * pair of query blocks (128 rows; 256 for d_qk = 192; an odd count rounded up)
 * two block slots, and per slot, range and row an fp32 (max, sum) pair for
 * each of the row's two lanes and d_v fp32 partial outputs.  0 for n_split <=
 * 1, n_split above 16 or an unsupported head-dim pair. */
size_t mha_fwd_bf16_split_workspace_bytes(int b, int hq, int sq, int d_qk, int d_v, int n_split);

/* The n_split for this shape on the CURRENT device (its compute units): 1 when
 * the unsplit grid keeps the device busy and for empty shapes; otherwise the
 * split (2..8) that a time model (workgroups per CU, a lone 4-wave workgroup at
 * 0.87 of a CU's two-wave throughput, the merge's fp32 partial traffic)
 * predicts at least 10% faster, among those whose ranges keep keys * (d_qk +
 * d_v) >= 2^18 (fixed costs dominate below).  Shape errors as mha_fwd_bf16;
 * MHA_ERR_HIP if the device cannot be queried (then *n_split = 1). */
mha_status mha_fwd_bf16_split_plan(int b, int hq, int hk, int sq, int sk, int d_qk, int d_v, int causal,
                                   int* n_split);

/*
 * mha_fwd_bf16_window_sink - mha_fwd_bf16 with a sliding window and per-head
 * attention sinks: the GPT-OSS "sink+sliding-window" shapes named in the Test
 * Result section of "Tune MHA config & small-head pipeline pathology".
 *
 *   window_left, window_right  query i sees key j only if j >= i - window_left
 *       and j <= i + window_right, on top of the causal rule; -1 leaves that
 *       side unbounded (a 128-token causal window is window_left = 127);
 *       values below -1 are refused (MHA_ERR_VALUE)
 *   sinks  [hq] fp32 device array of per-query-head logits in the units of
 *       the scaled scores, or NULL: each joins its head's softmax normaliser
 *       without a value row, O_i = sum_j e^(s_ij - m) v_j / (sum_j e^(s_ij - m)
 *       + e^(sink_h - m)), and LSE includes it; 4-byte aligned
 * Everything else (shapes, layouts, errors) as mha_fwd_bf16.  Key tiles left of
 * a query block's window are never loaded.  A row that sees no key gets O = 0
 * and LSE = sink_h (-inf without sinks).
 */
mha_status mha_fwd_bf16_window_sink(const void* q, mha_strides q_stride,
                                    const void* k, mha_strides k_stride,
                                    const void* v, mha_strides v_stride,
                                    void* o, mha_strides o_stride,
                                    float* lse,
                                    int b, int hq, int hk, int sq, int sk, int d_qk, int d_v,
                                    float softmax_scale, int causal,
                                    int window_left, int window_right, const float* sinks,
                                    void* stream);

/*
 * mha_fwd_bf16_varlen - mha_fwd_bf16 over a batch of packed sequences of
 * different lengths: the "varlen" layout the retuned Triton MHA forward is
 * timed in next to BSHD ("Tune MHA config & small-head pipeline pathology",
 * Test Plan and the per-shape tables' layout column).
 *
 *   q    [total_q, hq, d_qk] bf16      k [total_k, hk, d_qk] bf16
 *   v    [total_k, hk, d_v]  bf16      o [total_q, hq, d_v]  bf16 (written)
 *   lse  [hq, total_q] fp32 contiguous (written), or NULL
 *   cu_seqlens_q, cu_seqlens_k: device int32 arrays of b + 1 entries; sequence
 *        i owns query tokens [cu_seqlens_q[i], cu_seqlens_q[i+1]) and key tokens
 *        [cu_seqlens_k[i], cu_seqlens_k[i+1]).  The caller guarantees
 *        0 = cu[0] <= cu[1] <= ... <= cu[b] = total and that every length is
 *        at most max_seqlen_q / max_seqlen_k (query rows past max_seqlen_q would
 *        be left unwritten).  The kernel clamps offsets to [0, total] and lengths
 *        to the maxima, so inconsistent arrays give wrong values but never an
 *        access outside q, k, v, o or lse.
 *   A sequence without keys gives O = 0 and LSE = -inf on its rows.
 *   causal: within a sequence, key j is visible to query i iff j <= i (top-left).
 *   Strides: token stride .s and head stride .h; .b is ignored.  Layout and
 *   size rules as mha_fwd_bf16 with the packed token axis as the one batch row
 *   (the whole packed tensor must span < 2^31 bytes per head).
 */
mha_status mha_fwd_bf16_varlen(const void* q, mha_strides q_stride,
                               const void* k, mha_strides k_stride,
                               const void* v, mha_strides v_stride,
                               void* o, mha_strides o_stride,
                               float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int b, int hq, int hk, int total_q, int total_k,
                               int max_seqlen_q, int max_seqlen_k, int d_qk, int d_v,
                               float softmax_scale, int causal, void* stream);

/*
 * mha_fwd_bf16_varlen_window_sink - mha_fwd_bf16_varlen with the sliding window
 * and per-head sinks of mha_fwd_bf16_window_sink (the GPT-OSS shapes are
 * served packed): window positions are counted inside each sequence, sinks
 * is a [hq] fp32 device array or NULL.  Arguments, layouts and errors as the
 * two calls it combines.
 */
mha_status mha_fwd_bf16_varlen_window_sink(const void* q, mha_strides q_stride,
                                           const void* k, mha_strides k_stride,
                                           const void* v, mha_strides v_stride,
                                           void* o, mha_strides o_stride,
                                           float* lse,
                                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                           int b, int hq, int hk, int total_q, int total_k,
                                           int max_seqlen_q, int max_seqlen_k, int d_qk, int d_v,
                                           float softmax_scale, int causal,
                                           int window_left, int window_right, const float* sinks,
                                           void* stream);

/*
 * k_smooth_mean - the K-smoothing gate of "[HIP] Mha v4: run the K-smoothing
 * gate as one HIP call" (Summary; commit message): per-(batch*kv head, chunk)
 * moments over a strided key sample, then a per-head fold and a threshold,
 * as two deterministic kernels behind one call.
 *
 *   k           [b, sk, hk, d] bf16 view (any 2-byte alignment; misaligned
 *               views take a scalar-load path)
 *   key_stride  >= 1: keys 0, key_stride, 2*key_stride, ... are sampled
 *   max_keys    >= 0: at most this many samples (0 = no cap)
 *   tau         gate threshold (finite)
 *   mean        [b, hk, d] fp32 contiguous (written): the per-channel sample
 *               mean mu where the gate is open, exactly 0 where it is closed
 *   gate        [b, hk] int32 contiguous (written) 1 = open, 0 = closed, or NULL
 *   ws          device workspace of at least k_smooth_mean_workspace_bytes(),
 *               256-byte aligned; its contents on entry do not matter
 *   d in {64, 128, 256}; b, sk >= 0; hk >= 1.
 *
 * Statistic: over T samples (T = ceil(sk / key_stride), capped at max_keys),
 * mu_c = sum x / T, var_c = max(sum x^2 / T - mu_c^2, 0) in fp32 (sums kept in
 * fp32, in a fixed order); r = sqrt(sum_c mu_c^2 / sum_c var_c) (r = +inf when
 * the variance sum is 0 and the mean sum is not, 0 when both are 0); the gate
 * is open iff r > tau.  T == 0 gives a closed gate and zero mean.
 */
size_t k_smooth_mean_workspace_bytes(int b, int hk, int sk, int d, int key_stride, int max_keys);

mha_status k_smooth_mean(const void* k, mha_strides k_stride,
                         int b, int hk, int sk, int d, int key_stride, int max_keys, float tau,
                         float* mean, int32_t* gate,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * k_smooth_mean_noalloc - k_smooth_mean without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * Same arguments, results and errors as k_smooth_mean, minus ws / ws_bytes: the per-chunk
 * moments go to a scratch array the library holds in each GPU's memory (4 MiB per GPU, kept
 * until the process ends).  It allocates nothing.  Calls whose moments need more than 4 MiB,
 * i.e. k_smooth_mean_workspace_bytes(...) > 4194304 (b * hk * ceil(T / 256) * 2 * d * 4 bytes,
 * T the sample count), are refused with MHA_ERR_WORKSPACE and launch nothing.
 * Every call on one GPU shares that GPU's scratch, whatever the stream: calls that overlap
 * in time on one GPU (concurrent streams, host threads) race and may give wrong results;
 * calls in one stream order are safe.  The scratch needs no clearing: each call overwrites
 * every moment it reads.
 */
mha_status k_smooth_mean_noalloc(const void* k, mha_strides k_stride,
                                 int b, int hk, int sk, int d,
                                 int key_stride, int max_keys, float tau,
                                 float* mean, int32_t* gate, void* stream);

/*
 * mha_fwd_fp8 - attention forward on E4M3-quantised, K-smoothed inputs: the
 * quantised mha_v4 call with the FP8 hd128 recipe of "[HIP] Mha v4: run the
 * K-smoothing gate as one HIP call" (Performance table) and "MHA v4: fixes,
 * refactor, new kernel, perf tweaks" (BF16/FP8 recipe).
 *
 *   q [b, sq, hq, d], k [b, sk, hk, d], v [b, sk, hk, d]: bf16 views with the
 *     same layout requirements as mha_fwd_bf16
 *   k_mean  [b, hk, d] fp32 contiguous (usually k_smooth_mean's output), or
 *           NULL for no smoothing
 *   o [b, sq, hq, d] bf16 (written); lse [b, hq, sq] fp32 or NULL
 *   d in {64, 128} (the pages time hd128); softmax_scale finite; causal 0 or 1
 *   ws  device workspace of at least mha_fwd_fp8_workspace_bytes(), 256-byte
 *       aligned
 *
 * Steps: x_Q = fp32(Q), x_K = fp32(fp32(K) - k_mean), x_V = fp32(V); per
 * (batch, head, block of 128 tokens): amax = max |x|, scale = amax / 448 in
 * fp32 (1 when amax == 0), code = E4M3(x / scale) (OCP E4M3, round to nearest
 * even, saturating at +-448).  Scores are computed on the codes with fp8 MFMA
 * and rescaled by both block scales in fp32; P.V runs on bf16 MFMA with P
 * rounded to bf16 and the E4M3 V codes widened exactly; the V block scale is
 * applied in fp32.  O is rounded to bf16 once.
 *
 * Workspace layout (byte offsets from ws; nblk_q = ceil(sq/128), nblk_k =
 * ceil(sk/128); every region starts 256-byte aligned):
 *   q codes   uint8 [b, hq, nblk_q*128, d]     (token-padded, zero-filled tail)
 *   k codes   uint8 [b, hk, nblk_k*128, d]
 *   v values  bf16  [b, hk, nblk_k*128, d]  (the E4M3 codes' values, widened exactly)
 *   q scales  fp32  [b, hq, nblk_q]
 *   k scales  fp32  [b, hk, nblk_k]
 *   v scales  fp32  [b, hk, nblk_k]
 * mha_fp8_workspace_layout() reports the six offsets so callers can read the
 * quantised tensors back.
 */
size_t mha_fwd_fp8_workspace_bytes(int b, int hq, int hk, int sq, int sk, int d);

/* Byte offsets of the six workspace regions above, in the order listed
 * (q codes, k codes, v values, q scales, k scales, v scales); returns
 * MHA_ERR_SHAPE for invalid sizes. `offsets` is a host array of 6. */
mha_status mha_fp8_workspace_layout(int b, int hq, int hk, int sq, int sk, int d, size_t* offsets);

mha_status mha_fwd_fp8(const void* q, mha_strides q_stride,
                       const void* k, mha_strides k_stride,
                       const void* v, mha_strides v_stride,
                       const float* k_mean,
                       void* o, mha_strides o_stride,
                       float* lse,
                       int b, int hq, int hk, int sq, int sk, int d,
                       float softmax_scale, int causal,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * mha_fwd_mxfp8 - the same quantised call with the MXFP8 hd128 recipe of
 * "[HIP] Mha v4: run the K-smoothing gate as one HIP call" (commit message
 * table) and its uint8 E8M0 per-1x32 descales ("MHA v4: fixes, refactor, new
 * kernel, perf tweaks", review comments), in the block format of OCP
 * Microscaling v1.0.  Arguments, layouts and errors as mha_fwd_fp8; the
 * workspace is sized by mha_fwd_mxfp8_workspace_bytes().
 *
 * Steps: x as for mha_fwd_fp8 (K smoothed by k_mean); every 32 channels of a
 * token row share an exponent E = clamp(floor(log2(amax)) - 8, -127, 127)
 * (E = -127 for a block of zeros), code = E4M3(x * 2^-E) (round to nearest
 * even, saturating at +-448).  Scores come from the fp8 MFMA with the Q and K
 * exponents as its per-block scale operands, so no fp32 rescaling follows;
 * V is kept as decode(code) * 2^E in bf16 (exact while in bf16's normal
 * range) and P.V runs on bf16 MFMA with P rounded to bf16.
 *
 * Workspace layout (byte offsets from ws, 256-byte aligned regions):
 *   q codes  uint8 [b, hq, nblk_q*128, d]    (token-padded, zero-filled tail)
 *   k codes  uint8 [b, hk, nblk_k*128, d]
 *   v values bf16  [b, hk, nblk_k*128, d]    (decode(code) * 2^E)
 *   q exps   uint8 [b, hq, nblk_q*128, d/32] (E8M0 bytes E + 127; tail rows 0)
 *   k exps   uint8 [b, hk, nblk_k*128, d/32]
 */
size_t mha_fwd_mxfp8_workspace_bytes(int b, int hq, int hk, int sq, int sk, int d);

/* Byte offsets of the five regions above, in the order listed; MHA_ERR_SHAPE for
 * invalid sizes (d must be a positive multiple of 32). `offsets` is a host array of 5. */
mha_status mha_mxfp8_workspace_layout(int b, int hq, int hk, int sq, int sk, int d, size_t* offsets);

mha_status mha_fwd_mxfp8(const void* q, mha_strides q_stride,
                         const void* k, mha_strides k_stride,
                         const void* v, mha_strides v_stride,
                         const float* k_mean,
                         void* o, mha_strides o_stride,
                         float* lse,
                         int b, int hq, int hk, int sq, int sk, int d,
                         float softmax_scale, int causal,
                         void* ws, size_t ws_bytes, void* stream);

/* Static string naming a status code. */
const char* mha_status_string(mha_status status);

/* Thread-local message of the last refusal or failure on this thread ("" if none). */
const char* mha_last_error(void);

/*
 * mha_debug_sync_enabled - whether the debug synchronisation switch is on (1) or off (0).
 *
 * The switch is the environment variable MHA_DEBUG_SYNC, read once, at the first call into the
 * library that needs it: any value other than "" or "0" turns it on.  Then every entry point
 * synchronises its stream after each kernel it launches and returns MHA_ERR_HIP, naming the
 * kernel, if that kernel failed while running.  Without it a kernel fault only surfaces at a
 * later synchronisation, often inside an unrelated launch: the failure mode described in
 * "MHA v4: fixes, refactor, new kernel, perf tweaks" (review comments, faults that surface
 * asynchronously in a later launch).  Costs one stream synchronisation per kernel; for
 * debugging only.
 */
int mha_debug_sync_enabled(void);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H_ */
