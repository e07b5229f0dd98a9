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
};

// Workgroups of `kernel` (launched with `threads` threads, no dynamic LDS) that the current
// device holds at once: CUs x resident workgroups per CU.  Cached per device and kernel.
hipError_t resident_groups(const void* kernel, int threads, int* groups);

// bf16 attention forward: d_qk/d_v in {(64,64), (128,128), (192,128)}.
hipError_t launch_attn_fwd_bf16(const AttnParams& p, int d_qk, int d_v, bool causal, hipStream_t stream);

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
