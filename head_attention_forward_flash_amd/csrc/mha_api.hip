// Host side of libmha: argument validation, workspace carving and the C ABI
// declared in include/mha.h.  Every check runs before any launch; a refusal
// launches nothing and records a message naming the argument.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mha.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

mha_status fail(mha_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

mha_status ok() {
    g_last_error.clear();
    return MHA_OK;
}

// MHA_DEBUG_SYNC, read once per process: set to anything but "" or "0", every launch is
// followed by a synchronisation of its stream, so that a kernel fault is reported by the call
// that launched the kernel instead of surfacing in a later, unrelated one.
bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("MHA_DEBUG_SYNC");
        return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
    }();
    return on;
}

// Status of a launch just enqueued on `stream` (with MHA_DEBUG_SYNC, of its execution too).
mha_status launched(hipError_t e, const char* what, void* stream) {
    if (e != hipSuccess) return fail(MHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    if (debug_sync()) {
        e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess)
            return fail(MHA_ERR_HIP, "%s: failed in execution (MHA_DEBUG_SYNC): %s", what, hipGetErrorString(e));
    }
    return ok();
}

constexpr int64_t kMaxSliceBytes = int64_t(1) << 31;

// Validates one BSHD view of `rows` rows and `d` channels of `elem` bytes and fills `out`.
// `vec_align`: require 16-byte aligned base and rows (vector-load kernels).
mha_status make_view(const char* name, const void* ptr, const mha_strides& st, int heads, int rows, int d,
                     int elem, bool vec_align, mha::View* out) {
    if (st.b < 0 || st.s < 0 || st.h < 0)
        return fail(MHA_ERR_LAYOUT, "%s: strides must be non-negative (b=%lld s=%lld h=%lld)", name,
                    (long long)st.b, (long long)st.s, (long long)st.h);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(ptr);
    if (addr % elem != 0) return fail(MHA_ERR_LAYOUT, "%s: pointer is not %d-byte aligned", name, elem);
    if (vec_align) {
        if (addr % 16 != 0) return fail(MHA_ERR_LAYOUT, "%s: pointer must be 16-byte aligned", name);
        const int64_t per16 = 16 / elem;
        if (st.b % per16 || st.s % per16 || st.h % per16)
            return fail(MHA_ERR_LAYOUT, "%s: strides must be multiples of %lld elements (b=%lld s=%lld h=%lld)",
                        name, (long long)per16, (long long)st.b, (long long)st.s, (long long)st.h);
    }
    int64_t slice = 0;
    if (rows > 0) {
        if (st.s > 0 && (rows - 1) > (kMaxSliceBytes / elem) / st.s)
            return fail(MHA_ERR_OVERFLOW, "%s: one (batch, head) slice spans >= 2^31 bytes (stride.s=%lld, rows=%d)",
                        name, (long long)st.s, rows);
        slice = ((int64_t)(rows - 1) * st.s + d) * elem;
        if (slice >= kMaxSliceBytes)
            return fail(MHA_ERR_OVERFLOW, "%s: one (batch, head) slice spans >= 2^31 bytes", name);
    }
    (void)heads;
    out->sb = st.b;
    out->ss = st.s;
    out->sh = st.h;
    out->slice_bytes = static_cast<uint32_t>(slice);
    return MHA_OK;
}

bool supported_bf16(int dqk, int dv) {
    return (dqk == 32 && dv == 32) || (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) ||
           (dqk == 192 && dv == 128);
}

mha_status check_common(int b, int hq, int hk, int sq, int sk, float scale, int causal) {
    if (b < 0 || sq < 0 || sk < 0) return fail(MHA_ERR_SHAPE, "b, sq, sk must be >= 0 (b=%d sq=%d sk=%d)", b, sq, sk);
    if (hq < 1 || hk < 1) return fail(MHA_ERR_SHAPE, "hq, hk must be >= 1 (hq=%d hk=%d)", hq, hk);
    if (hq % hk != 0) return fail(MHA_ERR_SHAPE, "hq (%d) must be a multiple of hk (%d)", hq, hk);
    if (!std::isfinite(scale)) return fail(MHA_ERR_VALUE, "softmax_scale must be finite");
    if (causal != 0 && causal != 1) return fail(MHA_ERR_VALUE, "causal must be 0 or 1 (got %d)", causal);
    return MHA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kMaxSplit = 16;   // key ranges per query block of the split call

}  // namespace

extern "C" {

const char* mha_status_string(mha_status s) {
    switch (s) {
        case MHA_OK: return "MHA_OK";
        case MHA_ERR_NULL: return "MHA_ERR_NULL";
        case MHA_ERR_SHAPE: return "MHA_ERR_SHAPE";
        case MHA_ERR_UNSUPPORTED: return "MHA_ERR_UNSUPPORTED";
        case MHA_ERR_LAYOUT: return "MHA_ERR_LAYOUT";
        case MHA_ERR_OVERFLOW: return "MHA_ERR_OVERFLOW";
        case MHA_ERR_WORKSPACE: return "MHA_ERR_WORKSPACE";
        case MHA_ERR_HIP: return "MHA_ERR_HIP";
        case MHA_ERR_VALUE: return "MHA_ERR_VALUE";
    }
    return "MHA_ERR_UNKNOWN";
}

const char* mha_last_error(void) { return g_last_error.c_str(); }

int mha_debug_sync_enabled(void) { return debug_sync() ? 1 : 0; }

}  // extern "C"

namespace {

mha_status fwd_bf16(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride, const void* v,
                    mha_strides v_stride, void* o, mha_strides o_stride, float* lse, int b, int hq, int hk, int sq,
                    int sk, int d_qk, int d_v, float softmax_scale, int causal, int window_left, int window_right,
                    const float* sinks, int n_split, void* ws, size_t ws_bytes, void* stream) {
    mha_status st = check_common(b, hq, hk, sq, sk, softmax_scale, causal);
    if (st != MHA_OK) return st;
    if (window_left < -1 || window_right < -1)
        return fail(MHA_ERR_VALUE, "window_left = %d, window_right = %d: each must be >= -1 (-1 = unbounded)",
                    window_left, window_right);
    if (sinks && reinterpret_cast<uintptr_t>(sinks) % 4 != 0) return fail(MHA_ERR_LAYOUT, "sinks must be 4-byte aligned");
    if (!supported_bf16(d_qk, d_v))
        return fail(MHA_ERR_UNSUPPORTED, "(d_qk, d_v) = (%d, %d) not built; supported: (32,32) (64,64) (128,128) (192,128)",
                    d_qk, d_v);
    // Empty problems need no memory: q/o may be NULL when there are no query rows, k/v when
    // there are no keys.
    const bool has_rows = b > 0 && sq > 0;
    if (has_rows && !q) return fail(MHA_ERR_NULL, "q is NULL");
    if (has_rows && sk > 0 && !k) return fail(MHA_ERR_NULL, "k is NULL");
    if (has_rows && sk > 0 && !v) return fail(MHA_ERR_NULL, "v is NULL");
    if (has_rows && !o) return fail(MHA_ERR_NULL, "o is NULL");
    if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0) return fail(MHA_ERR_LAYOUT, "lse must be 4-byte aligned");

    mha::AttnParams p{};
    if ((st = make_view("q", q, q_stride, hq, sq, d_qk, 2, true, &p.qv)) != MHA_OK) return st;
    if ((st = make_view("k", k, k_stride, hk, sk, d_qk, 2, true, &p.kv)) != MHA_OK) return st;
    if ((st = make_view("v", v, v_stride, hk, sk, d_v, 2, true, &p.vv)) != MHA_OK) return st;
    if ((st = make_view("o", o, o_stride, hq, sq, d_v, 2, true, &p.ov)) != MHA_OK) return st;
    // The kernel zero-fills keys past sk by bounding each tile's loads at the slice end, which
    // needs key rows that do not overlap.
    if (sk > 1 && k_stride.s < d_qk)
        return fail(MHA_ERR_LAYOUT, "k: rows overlap (stride.s = %lld < d_qk = %d)", (long long)k_stride.s, d_qk);
    if (sk > 1 && v_stride.s < d_v)
        return fail(MHA_ERR_LAYOUT, "v: rows overlap (stride.s = %lld < d_v = %d)", (long long)v_stride.s, d_v);

    // the launcher sizes the grid from its tile configuration (at least 128 rows per workgroup)
    const int64_t nwg = int64_t(b) * hq * ((int64_t(sq) + 127) / 128);
    if (nwg > INT32_MAX) return fail(MHA_ERR_OVERFLOW, "grid of %lld workgroups exceeds 2^31-1", (long long)nwg);
    if (nwg == 0) return ok();

    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.b = b;
    p.hq = hq;
    p.hk = hk;
    p.sq = sq;
    p.sk = sk;
    p.group = hq / hk;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    // a side of the window that reaches past every key is no bound at all
    p.window_left = window_left >= sq ? -1 : window_left;
    p.window_right = (causal || window_right >= sk) ? -1 : window_right;
    p.sinks = sinks;
    if (n_split < 1 || n_split > kMaxSplit)
        return fail(MHA_ERR_VALUE, "n_split = %d: must be in [1, %d]", n_split, kMaxSplit);
    if (n_split > 1) {
        if (window_left >= 0 || window_right >= 0 || sinks)
            return fail(MHA_ERR_UNSUPPORTED, "the key-range split takes no window or sinks");
        const int most = mha::attn_bf16_split_max(sq, sk, d_qk, d_v, causal != 0);
        if (n_split > most)
            return fail(MHA_ERR_VALUE, "n_split = %d exceeds the %d key tiles of 64 that the shortest %s holds (sk = %d)",
                        n_split, most, causal ? "pair of causal query blocks" : "query block", sk);
        size_t off[2];
        const size_t need = mha::attn_bf16_split_layout(b, hq, sq, d_qk, d_v, n_split, off);
        if (!ws) return fail(MHA_ERR_WORKSPACE, "ws is NULL (need %zu bytes)", need);
        if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MHA_ERR_WORKSPACE, "ws must be 256-byte aligned");
        if (ws_bytes < need) return fail(MHA_ERR_WORKSPACE, "ws_bytes = %zu < required %zu", ws_bytes, need);
        char* w = static_cast<char*>(ws);
        p.n_split = n_split;
        p.split_ml = reinterpret_cast<float*>(w + off[0]);
        p.split_o = reinterpret_cast<float*>(w + off[1]);
    }
    return launched(mha::launch_attn_fwd_bf16(p, d_qk, d_v, causal != 0, static_cast<hipStream_t>(stream)),
                    "attn_fwd_bf16", stream);
}

}  // namespace

extern "C" {

mha_status mha_fwd_bf16(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride,
                        const void* v, mha_strides v_stride, void* o, mha_strides o_stride, float* lse,
                        int b, int hq, int hk, int sq, int sk, int d_qk, int d_v, float softmax_scale,
                        int causal, void* stream) {
    return fwd_bf16(q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, b, hq, hk, sq, sk, d_qk, d_v,
                    softmax_scale, causal, -1, -1, nullptr, 1, nullptr, 0, stream);
}

mha_status mha_fwd_bf16_split_plan(int b, int hq, int hk, int sq, int sk, int d_qk, int d_v, int causal,
                                   int* n_split) {
    if (!n_split) return fail(MHA_ERR_NULL, "n_split is NULL");
    *n_split = 1;
    mha_status st = check_common(b, hq, hk, sq, sk, 1.f, causal);
    if (st != MHA_OK) return st;
    if (!supported_bf16(d_qk, d_v))
        return fail(MHA_ERR_UNSUPPORTED, "(d_qk, d_v) = (%d, %d) not built; supported: (32,32) (64,64) (128,128) (192,128)",
                    d_qk, d_v);
    const hipError_t e = mha::attn_bf16_split_plan(b, hq, sq, sk, d_qk, d_v, causal != 0, n_split);
    if (e != hipSuccess) {
        *n_split = 1;
        return fail(MHA_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
    }
    return ok();
}

size_t mha_fwd_bf16_split_workspace_bytes(int b, int hq, int sq, int d_qk, int d_v, int n_split) {
    if (n_split <= 1 || n_split > kMaxSplit) return 0;
    size_t off[2];
    return mha::attn_bf16_split_layout(b, hq, sq, d_qk, d_v, n_split, off);
}

mha_status mha_fwd_bf16_split(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride,
                              const void* v, mha_strides v_stride, void* o, mha_strides o_stride, float* lse,
                              int b, int hq, int hk, int sq, int sk, int d_qk, int d_v, float softmax_scale,
                              int causal, int n_split, void* ws, size_t ws_bytes, void* stream) {
    return fwd_bf16(q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, b, hq, hk, sq, sk, d_qk, d_v,
                    softmax_scale, causal, -1, -1, nullptr, n_split, ws, ws_bytes, stream);
}

mha_status mha_fwd_bf16_window_sink(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride,
                                    const void* v, mha_strides v_stride, void* o, mha_strides o_stride, float* lse,
                                    int b, int hq, int hk, int sq, int sk, int d_qk, int d_v, float softmax_scale,
                                    int causal, int window_left, int window_right, const float* sinks,
                                    void* stream) {
    return fwd_bf16(q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, b, hq, hk, sq, sk, d_qk, d_v,
                    softmax_scale, causal, window_left, window_right, sinks, 1, nullptr, 0, stream);
}

}  // extern "C"

namespace {

mha_status fwd_bf16_varlen(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride, const void* v,
                           mha_strides v_stride, void* o, mha_strides o_stride, float* lse,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int b, int hq, int hk,
                           int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d_qk, int d_v,
                           float softmax_scale, int causal, int window_left, int window_right, const float* sinks,
                           void* stream) {
    if (window_left < -1 || window_right < -1)
        return fail(MHA_ERR_VALUE, "window_left = %d, window_right = %d: each must be >= -1 (-1 = unbounded)",
                    window_left, window_right);
    if (sinks && reinterpret_cast<uintptr_t>(sinks) % 4 != 0) return fail(MHA_ERR_LAYOUT, "sinks must be 4-byte aligned");
    if (total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(MHA_ERR_SHAPE, "total_q, total_k, max_seqlen_q, max_seqlen_k must be >= 0 (%d %d %d %d)",
                    total_q, total_k, max_seqlen_q, max_seqlen_k);
    mha_status st = check_common(b, hq, hk, max_seqlen_q, max_seqlen_k, softmax_scale, causal);
    if (st != MHA_OK) return st;
    if (!supported_bf16(d_qk, d_v))
        return fail(MHA_ERR_UNSUPPORTED, "(d_qk, d_v) = (%d, %d) not built; supported: (32,32) (64,64) (128,128) (192,128)",
                    d_qk, d_v);
    const bool has_rows = b > 0 && total_q > 0 && max_seqlen_q > 0;
    if (b > 0 && (!cu_seqlens_q || !cu_seqlens_k)) return fail(MHA_ERR_NULL, "cu_seqlens_q / cu_seqlens_k is NULL");
    if (reinterpret_cast<uintptr_t>(cu_seqlens_q) % 4 || reinterpret_cast<uintptr_t>(cu_seqlens_k) % 4)
        return fail(MHA_ERR_LAYOUT, "cu_seqlens arrays must be 4-byte aligned");
    if (has_rows && !q) return fail(MHA_ERR_NULL, "q is NULL");
    if (has_rows && total_k > 0 && !k) return fail(MHA_ERR_NULL, "k is NULL");
    if (has_rows && total_k > 0 && !v) return fail(MHA_ERR_NULL, "v is NULL");
    if (has_rows && !o) return fail(MHA_ERR_NULL, "o is NULL");
    if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0) return fail(MHA_ERR_LAYOUT, "lse must be 4-byte aligned");
    if (int64_t(hq) * total_q > INT32_MAX) return fail(MHA_ERR_OVERFLOW, "hq * total_q exceeds 2^31-1");

    // The packed token axis plays the role of one batch row: the batch stride is ignored.
    auto packed = [](mha_strides s) { return mha_strides{0, s.s, s.h}; };
    mha::AttnParams p{};
    if ((st = make_view("q", q, packed(q_stride), hq, total_q, d_qk, 2, true, &p.qv)) != MHA_OK) return st;
    if ((st = make_view("k", k, packed(k_stride), hk, total_k, d_qk, 2, true, &p.kv)) != MHA_OK) return st;
    if ((st = make_view("v", v, packed(v_stride), hk, total_k, d_v, 2, true, &p.vv)) != MHA_OK) return st;
    if ((st = make_view("o", o, packed(o_stride), hq, total_q, d_v, 2, true, &p.ov)) != MHA_OK) return st;
    if (total_k > 1 && k_stride.s < d_qk)
        return fail(MHA_ERR_LAYOUT, "k: rows overlap (stride.s = %lld < d_qk = %d)", (long long)k_stride.s, d_qk);
    if (total_k > 1 && v_stride.s < d_v)
        return fail(MHA_ERR_LAYOUT, "v: rows overlap (stride.s = %lld < d_v = %d)", (long long)v_stride.s, d_v);

    const int64_t nwg = int64_t(b) * hq * ((int64_t(max_seqlen_q) + 127) / 128);
    if (nwg > INT32_MAX) return fail(MHA_ERR_OVERFLOW, "grid of %lld workgroups exceeds 2^31-1", (long long)nwg);
    if (!has_rows) return ok();

    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.b = b;
    p.hq = hq;
    p.hk = hk;
    p.sq = max_seqlen_q;
    p.sk = max_seqlen_k;
    p.group = hq / hk;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.total_q = total_q;
    p.total_k = total_k;
    // a side of the window that reaches past every key of the longest sequence is no bound
    p.window_left = window_left >= max_seqlen_q ? -1 : window_left;
    p.window_right = (causal || window_right >= max_seqlen_k) ? -1 : window_right;
    p.sinks = sinks;
    return launched(mha::launch_attn_fwd_bf16(p, d_qk, d_v, causal != 0, static_cast<hipStream_t>(stream)),
                    "attn_fwd_bf16 (varlen)", stream);
}

}  // namespace

extern "C" {

mha_status mha_fwd_bf16_varlen(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride,
                               const void* v, mha_strides v_stride, void* o, mha_strides o_stride, float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int b, int hq, int hk,
                               int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d_qk, int d_v,
                               float softmax_scale, int causal, void* stream) {
    return fwd_bf16_varlen(q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, cu_seqlens_q, cu_seqlens_k, b, hq,
                           hk, total_q, total_k, max_seqlen_q, max_seqlen_k, d_qk, d_v, softmax_scale, causal, -1, -1,
                           nullptr, stream);
}

mha_status mha_fwd_bf16_varlen_window_sink(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride,
                                           const void* v, mha_strides v_stride, void* o, mha_strides o_stride,
                                           float* lse, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                           int b, int hq, int hk, int total_q, int total_k, int max_seqlen_q,
                                           int max_seqlen_k, int d_qk, int d_v, float softmax_scale, int causal,
                                           int window_left, int window_right, const float* sinks, void* stream) {
    return fwd_bf16_varlen(q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, cu_seqlens_q, cu_seqlens_k, b, hq,
                           hk, total_q, total_k, max_seqlen_q, max_seqlen_k, d_qk, d_v, softmax_scale, causal,
                           window_left, window_right, sinks, stream);
}

size_t k_smooth_mean_workspace_bytes(int b, int hk, int sk, int d, int key_stride, int max_keys) {
    if (b < 0 || hk < 1 || sk < 0 || d < 1 || key_stride < 1 || max_keys < 0) return 0;
    int64_t t = sk > 0 ? (int64_t(sk) + key_stride - 1) / key_stride : 0;
    if (max_keys > 0 && t > max_keys) t = max_keys;
    const int64_t chunks = (t + mha::kGateChunk - 1) / mha::kGateChunk;
    return align256(size_t(b) * hk * (chunks > 0 ? chunks : 1) * 2 * d * sizeof(float));
}

}  // extern "C"

// Scratch of k_smooth_mean_noalloc: the per-chunk moments live here instead of in a caller's
// workspace, for callers that cannot allocate.  One copy per GPU, held until the process ends;
// every call on a GPU shares it.
static constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_lock;
std::vector<void*> g_scratch_ptr;   // device address of `scratch`, per device id

// The device address of the current device's copy of `scratch`, looked up on the first call on
// that device (with that device current).  The array's name is a host-side stand-in: only this
// address may be handed to kernels.
mha_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MHA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> g(g_scratch_lock);
    if (dev >= static_cast<int>(g_scratch_ptr.size())) g_scratch_ptr.resize(dev + 1, nullptr);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(MHA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MHA_OK;
}

// The gate of both entry points: `ws` is the caller's workspace, or with `noalloc` the
// library's scratch (then ws / ws_bytes are ignored).
mha_status gate_call(const void* k, mha_strides k_stride, int b, int hk, int sk, int d, int key_stride,
                     int max_keys, float tau, float* mean, int32_t* gate, void* ws, size_t ws_bytes, bool noalloc,
                     void* stream) {
    if (b < 0 || sk < 0) return fail(MHA_ERR_SHAPE, "b, sk must be >= 0 (b=%d sk=%d)", b, sk);
    if (hk < 1) return fail(MHA_ERR_SHAPE, "hk must be >= 1 (hk=%d)", hk);
    if (d != 64 && d != 128 && d != 256) return fail(MHA_ERR_UNSUPPORTED, "d = %d not built; supported: 64 128 256", d);
    if (key_stride < 1) return fail(MHA_ERR_VALUE, "key_stride must be >= 1 (got %d)", key_stride);
    if (max_keys < 0) return fail(MHA_ERR_VALUE, "max_keys must be >= 0 (got %d)", max_keys);
    if (!std::isfinite(tau)) return fail(MHA_ERR_VALUE, "tau must be finite");
    if (!k && b > 0 && sk > 0) return fail(MHA_ERR_NULL, "k is NULL");
    if (!mean && b > 0) return fail(MHA_ERR_NULL, "mean is NULL");
    if (reinterpret_cast<uintptr_t>(mean) % 4) return fail(MHA_ERR_LAYOUT, "mean must be 4-byte aligned");
    if (gate && reinterpret_cast<uintptr_t>(gate) % 4) return fail(MHA_ERR_LAYOUT, "gate must be 4-byte aligned");
    if (b == 0) return ok();

    mha::GateParams p{};
    mha_status st = make_view("k", k, k_stride, hk, sk, d, 2, false, &p.kv);
    if (st != MHA_OK) return st;
    const size_t need = k_smooth_mean_workspace_bytes(b, hk, sk, d, key_stride, max_keys);
    if (noalloc) {
        if (need > kScratchBytes)
            return fail(MHA_ERR_WORKSPACE,
                        "the moments need %zu bytes of scratch, above the %zu bytes the library holds per GPU "
                        "(lower max_keys, or call k_smooth_mean with a workspace)", need, kScratchBytes);
        if ((st = scratch_address(&ws)) != MHA_OK) return st;
        ws_bytes = kScratchBytes;
    }
    if (!ws) return fail(MHA_ERR_WORKSPACE, "ws is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MHA_ERR_WORKSPACE, "ws must be 256-byte aligned");
    if (ws_bytes < need) return fail(MHA_ERR_WORKSPACE, "ws_bytes = %zu < required %zu", ws_bytes, need);

    int64_t t = sk > 0 ? (int64_t(sk) + key_stride - 1) / key_stride : 0;
    if (max_keys > 0 && t > max_keys) t = max_keys;
    const int64_t n_chunks = (t + mha::kGateChunk - 1) / mha::kGateChunk;
    if (n_chunks * b * hk > INT32_MAX)
        return fail(MHA_ERR_OVERFLOW, "gate grid of %lld workgroups exceeds 2^31-1", (long long)(n_chunks * b * hk));
    const uintptr_t kaddr = reinterpret_cast<uintptr_t>(k);
    p.k = k;
    p.b = b;
    p.hk = hk;
    p.sk = sk;
    p.d = d;
    p.key_stride = key_stride;
    p.n_samples = static_cast<int>(t);
    p.n_chunks = static_cast<int>((t + mha::kGateChunk - 1) / mha::kGateChunk);
    p.tau = tau;
    p.partial = static_cast<float*>(ws);
    p.mean = mean;
    p.gate = gate;
    p.aligned = (kaddr % 16 == 0) && (k_stride.b % 8 == 0) && (k_stride.s % 8 == 0) && (k_stride.h % 8 == 0);
    return launched(mha::launch_k_smooth_mean(p, static_cast<hipStream_t>(stream)), "k_moments / k_fold_gate", stream);
}

}  // namespace

extern "C" {

mha_status k_smooth_mean(const void* k, mha_strides k_stride, int b, int hk, int sk, int d, int key_stride,
                         int max_keys, float tau, float* mean, int32_t* gate, void* ws, size_t ws_bytes,
                         void* stream) {
    return gate_call(k, k_stride, b, hk, sk, d, key_stride, max_keys, tau, mean, gate, ws, ws_bytes, false, stream);
}

mha_status k_smooth_mean_noalloc(const void* k, mha_strides k_stride, int b, int hk, int sk, int d, int key_stride,
                                 int max_keys, float tau, float* mean, int32_t* gate, void* stream) {
    return gate_call(k, k_stride, b, hk, sk, d, key_stride, max_keys, tau, mean, gate, nullptr, 0, true, stream);
}

mha_status mha_fp8_workspace_layout(int b, int hq, int hk, int sq, int sk, int d, size_t* offsets) {
    if (!offsets) return fail(MHA_ERR_NULL, "offsets is NULL");
    if (b < 0 || hq < 1 || hk < 1 || sq < 0 || sk < 0 || d < 1)
        return fail(MHA_ERR_SHAPE, "invalid sizes for the fp8 workspace");
    const size_t nq = (size_t(sq) + 127) / 128, nk = (size_t(sk) + 127) / 128;
    size_t off = 0;
    offsets[0] = off;
    off = align256(off + size_t(b) * hq * nq * 128 * d);
    offsets[1] = off;
    off = align256(off + size_t(b) * hk * nk * 128 * d);
    offsets[2] = off;
    off = align256(off + size_t(b) * hk * nk * 128 * d * 2);   // V values widened to bf16
    offsets[3] = off;
    off = align256(off + size_t(b) * hq * nq * 4);
    offsets[4] = off;
    off = align256(off + size_t(b) * hk * nk * 4);
    offsets[5] = off;
    return ok();
}

size_t mha_fwd_fp8_workspace_bytes(int b, int hq, int hk, int sq, int sk, int d) {
    size_t off[6];
    if (mha_fp8_workspace_layout(b, hq, hk, sq, sk, d, off) != MHA_OK) return 0;
    const size_t nk = (size_t(sk) + 127) / 128;
    return align256(off[5] + size_t(b) * hk * nk * 4);
}

mha_status mha_mxfp8_workspace_layout(int b, int hq, int hk, int sq, int sk, int d, size_t* offsets) {
    if (!offsets) return fail(MHA_ERR_NULL, "offsets is NULL");
    if (b < 0 || hq < 1 || hk < 1 || sq < 0 || sk < 0 || d < 32 || d % 32)
        return fail(MHA_ERR_SHAPE, "invalid sizes for the mxfp8 workspace");
    const size_t nq = (size_t(sq) + 127) / 128, nk = (size_t(sk) + 127) / 128;
    size_t off = 0;
    offsets[0] = off;
    off = align256(off + size_t(b) * hq * nq * 128 * d);
    offsets[1] = off;
    off = align256(off + size_t(b) * hk * nk * 128 * d);
    offsets[2] = off;
    off = align256(off + size_t(b) * hk * nk * 128 * d * 2);   // V values (2^E applied) in bf16
    offsets[3] = off;
    off = align256(off + size_t(b) * hq * nq * 128 * (d / 32));
    offsets[4] = off;
    return ok();
}

size_t mha_fwd_mxfp8_workspace_bytes(int b, int hq, int hk, int sq, int sk, int d) {
    size_t off[5];
    if (mha_mxfp8_workspace_layout(b, hq, hk, sq, sk, d, off) != MHA_OK) return 0;
    const size_t nk = (size_t(sk) + 127) / 128;
    return align256(off[4] + size_t(b) * hk * nk * 128 * (d / 32));
}

}  // extern "C"

namespace {

// The quantised call of both recipes: quantiser, then fp8 attention on its output.
mha_status fwd_quantised(bool mx, const void* q, mha_strides q_stride, const void* k, mha_strides k_stride,
                         const void* v, mha_strides v_stride, const float* k_mean, void* o, mha_strides o_stride,
                         float* lse, int b, int hq, int hk, int sq, int sk, int d, float softmax_scale, int causal,
                         void* ws, size_t ws_bytes, void* stream) {
    const char* name = mx ? "mxfp8" : "fp8";
    mha_status st = check_common(b, hq, hk, sq, sk, softmax_scale, causal);
    if (st != MHA_OK) return st;
    if (d != 64 && d != 128) return fail(MHA_ERR_UNSUPPORTED, "d = %d not built for %s; supported: 64 128", d, name);
    const bool has_rows = b > 0 && sq > 0;
    if (has_rows && !q) return fail(MHA_ERR_NULL, "q is NULL");
    if (has_rows && sk > 0 && !k) return fail(MHA_ERR_NULL, "k is NULL");
    if (has_rows && sk > 0 && !v) return fail(MHA_ERR_NULL, "v is NULL");
    if (has_rows && !o) return fail(MHA_ERR_NULL, "o is NULL");
    if (k_mean && reinterpret_cast<uintptr_t>(k_mean) % 4) return fail(MHA_ERR_LAYOUT, "k_mean must be 4-byte aligned");
    if (lse && reinterpret_cast<uintptr_t>(lse) % 4 != 0) return fail(MHA_ERR_LAYOUT, "lse must be 4-byte aligned");
    mha::View qv, kv, vv, ov;
    if ((st = make_view("q", q, q_stride, hq, sq, d, 2, true, &qv)) != MHA_OK) return st;
    if ((st = make_view("k", k, k_stride, hk, sk, d, 2, true, &kv)) != MHA_OK) return st;
    if ((st = make_view("v", v, v_stride, hk, sk, d, 2, true, &vv)) != MHA_OK) return st;
    if ((st = make_view("o", o, o_stride, hq, sq, d, 2, true, &ov)) != MHA_OK) return st;
    const size_t need = mx ? mha_fwd_mxfp8_workspace_bytes(b, hq, hk, sq, sk, d)
                           : mha_fwd_fp8_workspace_bytes(b, hq, hk, sq, sk, d);
    if (!ws) return fail(MHA_ERR_WORKSPACE, "ws is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MHA_ERR_WORKSPACE, "ws must be 256-byte aligned");
    if (ws_bytes < need) return fail(MHA_ERR_WORKSPACE, "ws_bytes = %zu < required %zu", ws_bytes, need);
    if (b == 0 || sq == 0) return ok();
    const int64_t nq = (int64_t(sq) + 127) / 128, nk = (int64_t(sk) + 127) / 128;
    if (std::max(nq, nk) * 128 * d * 2 >= kMaxSliceBytes)
        return fail(MHA_ERR_OVERFLOW, "%s: one (batch, head) slice of codes spans >= 2^31 bytes", name);
    const int64_t nwg = int64_t(b) * hq * nq;
    const int64_t nquant = int64_t(b) * (hq * nq + 2 * hk * nk);
    if (nwg > INT32_MAX || nquant > INT32_MAX)
        return fail(MHA_ERR_OVERFLOW, "%s: grid exceeds 2^31-1 workgroups", name);

    size_t off[6];
    if (mx)
        mha_mxfp8_workspace_layout(b, hq, hk, sq, sk, d, off);
    else
        mha_fp8_workspace_layout(b, hq, hk, sq, sk, d, off);
    char* wsb = static_cast<char*>(ws);
    auto quant = [&](const void* src, const mha::View& sv, const float* mean, int heads, int s, int64_t nblk,
                     size_t code_off, int64_t scale_off, bool widen) {
        mha::QuantParams qp{};
        qp.src = src;
        qp.sv = sv;
        qp.mean = mean;
        qp.b = b;
        qp.heads = heads;
        qp.s = s;
        qp.d = d;
        qp.nblk = static_cast<int>(nblk);
        qp.codes = reinterpret_cast<uint8_t*>(wsb + code_off);
        qp.mx = mx;
        if (mx)   // per-row exponents (V: none stored, its values carry them)
            qp.exps = scale_off >= 0 ? reinterpret_cast<uint8_t*>(wsb + scale_off) : nullptr;
        else
            qp.scales = reinterpret_cast<float*>(wsb + scale_off);
        qp.widen = widen;
        return qp;
    };
    mha::QuantParams qq, qk, qvv;
    if (mx) {
        qq = quant(q, qv, nullptr, hq, sq, nq, off[0], int64_t(off[3]), false);
        qk = quant(k, kv, k_mean, hk, sk, nk, off[1], int64_t(off[4]), false);
        qvv = quant(v, vv, nullptr, hk, sk, nk, off[2], -1, true);
    } else {
        qq = quant(q, qv, nullptr, hq, sq, nq, off[0], int64_t(off[3]), false);
        qk = quant(k, kv, k_mean, hk, sk, nk, off[1], int64_t(off[4]), false);
        qvv = quant(v, vv, nullptr, hk, sk, nk, off[2], int64_t(off[5]), true);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(mha::launch_quant_fp8(qq, qk, qvv, s), "quant_fp8", stream);
    if (st != MHA_OK) return st;

    mha::Fp8AttnParams p{};
    p.q = qq.codes;
    p.k = qk.codes;
    p.v = qvv.codes;
    p.q_scale = qq.scales;
    p.k_scale = qk.scales;
    p.v_scale = qvv.scales;
    if (mx) {
        p.q_exps = qq.exps;
        p.k_exps = qk.exps;
    }
    p.o = o;
    p.ov = ov;
    p.lse = lse;
    p.b = b;
    p.hq = hq;
    p.hk = hk;
    p.sq = sq;
    p.sk = sk;
    p.group = hq / hk;
    p.nq = static_cast<int>(nq);
    p.nk = static_cast<int>(nk);
    p.n_mblocks = static_cast<int>(nq);
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    return launched(mha::launch_attn_fwd_fp8(p, d, causal != 0, s), "attn_fwd_fp8", stream);
}

}  // namespace

extern "C" {

mha_status mha_fwd_fp8(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride, const void* v,
                       mha_strides v_stride, const float* k_mean, void* o, mha_strides o_stride, float* lse, int b,
                       int hq, int hk, int sq, int sk, int d, float softmax_scale, int causal, void* ws,
                       size_t ws_bytes, void* stream) {
    return fwd_quantised(false, q, q_stride, k, k_stride, v, v_stride, k_mean, o, o_stride, lse, b, hq, hk, sq, sk, d,
                         softmax_scale, causal, ws, ws_bytes, stream);
}

mha_status mha_fwd_mxfp8(const void* q, mha_strides q_stride, const void* k, mha_strides k_stride, const void* v,
                         mha_strides v_stride, const float* k_mean, void* o, mha_strides o_stride, float* lse, int b,
                         int hq, int hk, int sq, int sk, int d, float softmax_scale, int causal, void* ws,
                         size_t ws_bytes, void* stream) {
    return fwd_quantised(true, q, q_stride, k, k_stride, v, v_stride, k_mean, o, o_stride, lse, b, hq, hk, sq, sk, d,
                         softmax_scale, causal, ws, ws_bytes, stream);
}

}  // extern "C"
