// Kernel parameter blocks and host-side launchers of libmha (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

// One BSHD view: element strides (channel stride is 1) and the byte extent of
// one (batch, head) slice, which bounds every buffer load from that slice.
struct View {
    int64_t sb, ss, sh;
    uint32_t slice_bytes;
};

struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;      // may be null
    View qv, kv, vv, ov;
    int b, hq, hk, sq, sk;
    int group;       // hq / hk
    int n_mblocks;   // ceil(sq / rows per workgroup), set by the launcher
    float scale_log2;  // softmax_scale * log2(e)
    // packed sequences (varlen): b sequences, sequence i owning query tokens
    // [cu_q[i], cu_q[i+1]) and key tokens [cu_k[i], cu_k[i+1]) of a token axis of
    // total_q / total_k rows; sq / sk are then the maximum lengths.  cu_q == nullptr: dense.
    const int* cu_q = nullptr;
    const int* cu_k = nullptr;
    int total_q = 0, total_k = 0;
    // sliding window: query i sees keys i - window_left .. i + window_right (sequence positions),
    // -1 = unbounded on that side; per-query-head sink logits [hq] (nullptr = none)
    int window_left = -1, window_right = -1;
    const float* sinks = nullptr;
    // key-range split (dense grids): n_split workgroups per query block (causal: per pair of
    // blocks), each over a contiguous range of key tiles, leave their partial states in the
    // workspace below; a second kernel merges them.  n_split == 1: no split.
    int n_split = 1;
    float* split_ml = nullptr;    // [units, n_split, (causal: 2 blocks), waves, 64] (base-2 max, row sum)
    float* split_o = nullptr;     // [units, n_split, (causal: 2), waves, d_v / 32, 4, 64, 4] unnormalised O
};

// Workgroups of `kernel` (launched with `threads` threads, no dynamic LDS) that the current
// device holds at once: CUs x resident workgroups per CU.  Cached per device and kernel.
hipError_t resident_groups(const void* kernel, int threads, int* groups);

// bf16 attention forward: d_qk/d_v in {(32,32), (64,64), (128,128), (192,128)}.  With
// p.n_split > 1 (dense, non-causal, no window or sinks) the key-range split runs on the
// workspace pointers of p.
hipError_t launch_attn_fwd_bf16(const AttnParams& p, int d_qk, int d_v, bool causal, hipStream_t stream);

// Workspace of the key-range split: total bytes and the offsets of the (max, sum) and O regions
// (each 256-byte aligned).  0 for an unsupported head-dim pair.
size_t attn_bf16_split_layout(int b, int hq, int sq, int d_qk, int d_v, int n_split, size_t offsets[2]);

// Key ranges per query block (causal: per pair of blocks) that balance the grid of this shape on
// the current device (1: the unsplit grid already fills it, or the shape takes no split).
hipError_t attn_bf16_split_plan(int b, int hq, int sq, int sk, int d_qk, int d_v, bool causal, int* n_split);

// The largest n_split that leaves every range at least one key tile (0: no split possible).
int attn_bf16_split_max(int sq, int sk, int d_qk, int d_v, bool causal);

struct GateParams {
    const void* k;
    View kv;
    int b, hk, sk, d;
    int key_stride;
    int n_samples;   // T
    int n_chunks;    // ceil(T / chunk)
    float tau;
    float* partial;  // [b*hk, n_chunks, 2, d] fp32 workspace
    float* mean;     // [b, hk, d]
    int32_t* gate;   // [b, hk] or null
    bool aligned;    // 16-byte aligned rows: vector loads
};

constexpr int kGateChunk = 256;  // samples per moment chunk

hipError_t launch_k_smooth_mean(const GateParams& p, hipStream_t stream);

struct QuantParams {
    const void* src;
    View sv;
    const float* mean;  // [b, heads, d] subtracted before quantising, or null
    int b, heads, s, d;
    int nblk;            // ceil(s / 128)
    uint8_t* codes;      // [b, heads, nblk*128, d]: E4M3 codes, or with `widen` their values as bf16
    float* scales;       // [b, heads, nblk]
    bool widen;          // store each code's value widened (exactly) to bf16 instead of the byte
    bool mx;             // MXFP8: one E8M0 exponent per 32 channels of a token row instead of `scales`;
                         // widened values then include 2^E
    uint8_t* exps;       // MXFP8: [b, heads, nblk*128, d/32] E8M0 bytes, or null (not stored)
};

hipError_t launch_quant_fp8(const QuantParams& q, const QuantParams& k, const QuantParams& v,
                            hipStream_t stream);

struct Fp8AttnParams {
    const uint8_t* q;   // [b, hq, nq*128, d] codes
    const uint8_t* k;   // [b, hk, nk*128, d]
    const uint8_t* v;   // [b, hk, nk*128, d] bf16: the E4M3 codes' values, widened exactly
    const float* q_scale;  // [b, hq, nq]
    const float* k_scale;  // [b, hk, nk]
    const float* v_scale;  // [b, hk, nk]
    const uint8_t* q_exps = nullptr;   // MXFP8 when set: [b, hq, nq*128, 4] E8M0 bytes per 32 channels
    const uint8_t* k_exps = nullptr;   // [b, hk, nk*128, 4]; V then holds its values with 2^E applied
    void* o;
    View ov;
    float* lse;
    int b, hq, hk, sq, sk;
    int group;
    int nq, nk;          // token blocks of 128
    int n_mblocks;
    float scale_log2;
};

hipError_t launch_attn_fwd_fp8(const Fp8AttnParams& p, int d, bool causal, hipStream_t stream);

}  // namespace mha
