// K-smoothing gate: per-(batch, kv head) channel mean of K over a strided key
// sample, behind a threshold.  Two deterministic kernels behind one host call,
// as in "[HIP] Mha v4: run the K-smoothing gate as one HIP call" (Summary and
// commit message: per-(batch*head, chunk) moments over the strided sample, then
// a per-head fold and gate, within fp32 rounding of the former torch formula).
//
// Pass 1 (k_moments): one workgroup per (batch*kv head, chunk of 256 samples).
//   Threads split a sampled key row into 16-byte pieces (8 channels) and walk
//   the chunk's rows; per-thread fp32 sums of x and x^2 are then added across
//   the row groups in a fixed order through LDS.  Misaligned views load one
//   bf16 per thread instead.  Output: partial[bh][chunk][0|1][d].
// Pass 2 (k_fold_gate): one workgroup per batch*kv head.  Thread c folds its
//   channel's chunks in ascending order, forms mu and var, and a fixed-order
//   tree over channels gives sum mu^2 and sum var; the gate opens iff
//   sqrt(sum mu^2 / sum var) > tau.  Writes mean (mu or 0) and the flag.
//
// Both passes are HBM-/latency-bound; nothing here uses atomics, so results
// are bitwise reproducible.

#include "device_common.h"
#include "kernels.h"

namespace mha {
namespace {

constexpr int NT = 256;

template <int D, bool VEC>
__global__ __launch_bounds__(NT) void k_moments_kernel(const GateParams p) {
    constexpr int PER = VEC ? 8 : 1;          // channels per thread
    constexpr int TPR = D / PER;              // threads per sampled row
    constexpr int RG = NT / TPR;              // row groups in flight
    static_assert(NT % TPR == 0, "row split");
    __shared__ float red[2][RG][D];

    const int chunk = blockIdx.x % p.n_chunks;
    const int bh = blockIdx.x / p.n_chunks;
    const int bb = bh / p.hk, g = bh % p.hk;
    const char* base = static_cast<const char*>(p.k) + 2 * (bb * p.kv.sb + g * p.kv.sh);
    const auto rs = make_rsrc(base, p.kv.slice_bytes);

    const int tid = threadIdx.x;
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * PER;
    const int t_begin = chunk * kGateChunk;
    const int t_end = min(p.n_samples, t_begin + kGateChunk);

    float s1[PER], s2[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) s1[i] = s2[i] = 0.f;

    // The thread's rows t_begin + rg, + RG, ... are summed in that order.  All of a batch of
    // ROWS_IN_FLIGHT rows is loaded before any is added (rows past t_end read as zeros
    // through an out-of-range offset and are not added), so the loads overlap.
    constexpr int ROWS_IN_FLIGHT = kGateChunk / RG;
    for (int t0 = t_begin + rg; t0 < t_end; t0 += RG * ROWS_IN_FLIGHT) {
        if constexpr (VEC) {
            u32x4 w[ROWS_IN_FLIGHT];
#pragma unroll
            for (int j = 0; j < ROWS_IN_FLIGHT; ++j) {
                const int t = t0 + j * RG;
                const int64_t key = static_cast<int64_t>(t) * p.key_stride;
                const uint32_t off = t < t_end ? static_cast<uint32_t>((key * p.kv.ss + c0) * 2) : kOutOfRange;
                w[j] = buffer_load_b128(rs, off);
            }
#pragma unroll
            for (int j = 0; j < ROWS_IN_FLIGHT; ++j) {
                if (t0 + j * RG < t_end) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float lo = bf16_bits_to_float(w[j][i] & 0xffffu);
                        const float hi = bf16_bits_to_float(w[j][i] >> 16);
                        s1[2 * i] += lo;
                        s2[2 * i] += lo * lo;
                        s1[2 * i + 1] += hi;
                        s2[2 * i + 1] += hi * hi;
                    }
                }
            }
        } else {
            uint16_t w[ROWS_IN_FLIGHT];
#pragma unroll
            for (int j = 0; j < ROWS_IN_FLIGHT; ++j) {
                const int t = t0 + j * RG;
                const int64_t key = static_cast<int64_t>(t) * p.key_stride;
                const uint32_t off = t < t_end ? static_cast<uint32_t>((key * p.kv.ss + c0) * 2) : kOutOfRange;
                w[j] = buffer_load_b16(rs, off);
            }
#pragma unroll
            for (int j = 0; j < ROWS_IN_FLIGHT; ++j) {
                if (t0 + j * RG < t_end) {
                    const float x = bf16_bits_to_float(w[j]);
                    s1[0] += x;
                    s2[0] += x * x;
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        red[0][rg][c0 + i] = s1[i];
        red[1][rg][c0 + i] = s2[i];
    }
    __syncthreads();
    float* out = p.partial + (static_cast<int64_t>(bh) * p.n_chunks + chunk) * 2 * D;
    for (int idx = tid; idx < 2 * D; idx += NT) {
        const int which = idx / D, c = idx % D;
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) acc += red[which][r][c];
        out[idx] = acc;
    }
}

template <int D>
__global__ __launch_bounds__(NT) void k_fold_gate_kernel(const GateParams p) {
    __shared__ float num[NT];
    __shared__ float den[NT];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float inv_t = p.n_samples > 0 ? 1.f / static_cast<float>(p.n_samples) : 0.f;

    float mu = 0.f, var = 0.f;
    if (tid < D && p.n_samples > 0) {
        const float* src = p.partial + static_cast<int64_t>(bh) * p.n_chunks * 2 * D;
        float a = 0.f, b2 = 0.f;
        // ascending chunk order; sixteen chunks' partials are loaded before they are added
        constexpr int FOLD = 16;
        for (int c0 = 0; c0 < p.n_chunks; c0 += FOLD) {
            float pa[FOLD], pb[FOLD];
#pragma unroll
            for (int j = 0; j < FOLD; ++j) {
                const int c = min(c0 + j, p.n_chunks - 1);
                pa[j] = src[c * 2 * D + tid];
                pb[j] = src[c * 2 * D + D + tid];
            }
#pragma unroll
            for (int j = 0; j < FOLD; ++j) {
                if (c0 + j < p.n_chunks) {
                    a += pa[j];
                    b2 += pb[j];
                }
            }
        }
        mu = a / static_cast<float>(p.n_samples);
        var = fmaxf(b2 * inv_t - mu * mu, 0.f);
    }
    num[tid] = tid < D ? mu * mu : 0.f;
    den[tid] = tid < D ? var : 0.f;
    __syncthreads();
    // Pairwise tree over the NT slots: at level w, slot t < w adds slot t + w.  Levels whose
    // upper half lies past the D channels only add zeros and are skipped; levels w >= 64 pair
    // slots of different waves and go through LDS, the last six run inside each wave with lane
    // shuffles in the same pairing (every wave computes the same totals, so none has to wait
    // for another's).
#pragma unroll
    for (int w = NT / 2; w >= 64; w >>= 1) {
        if (w < D) {
            if (tid < w) {
                num[tid] += num[tid + w];
                den[tid] += den[tid + w];
            }
            __syncthreads();
        }
    }
    float sn = num[tid & 63], sd = den[tid & 63];
#pragma unroll
    for (int w = 32; w > 0; w >>= 1) {
        sn += __shfl_down(sn, w, 64);
        sd += __shfl_down(sd, w, 64);
    }
    sn = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sn)));
    sd = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sd)));
    float r;
    if (sd > 0.f) r = sqrtf(sn / sd);
    else r = sn > 0.f ? __builtin_inff() : 0.f;
    const bool open = r > p.tau;
    if (tid < D) p.mean[static_cast<int64_t>(bh) * D + tid] = open ? mu : 0.f;
    if (tid == 0 && p.gate != nullptr) p.gate[bh] = open ? 1 : 0;
}

template <int D>
hipError_t launch_d(const GateParams& p, hipStream_t stream) {
    const unsigned nbh = static_cast<unsigned>(p.b * p.hk);
    if (p.n_chunks > 0) {
        if (p.aligned)
            hipLaunchKernelGGL((k_moments_kernel<D, true>), dim3(p.n_chunks * nbh), dim3(NT), 0, stream, p);
        else
            hipLaunchKernelGGL((k_moments_kernel<D, false>), dim3(p.n_chunks * nbh), dim3(NT), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_fold_gate_kernel<D>), dim3(nbh), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_k_smooth_mean(const GateParams& p, hipStream_t stream) {
    switch (p.d) {
        case 64: return launch_d<64>(p, stream);
        case 128: return launch_d<128>(p, stream);
        case 256: return launch_d<256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mha
