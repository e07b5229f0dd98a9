// Device-side helpers shared by the gfx950 kernels of libmha.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr float kNegInf = -__builtin_inff();

// Byte offset that lies beyond every buffer extent the host accepts (< 2^31):
// a buffer load at this offset returns zeros instead of touching memory.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Raw buffer resource over [base, base + bytes); loads past `bytes` return 0.
// Word 3 (0x00020000) is the gfx9 raw-buffer configuration (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// A wave-uniform 64-bit value, moved through readfirstlane half by half so that the compiler
// keeps it (and a buffer descriptor built from it) in scalar registers.  readfirstlane
// returns a signed int: each half goes back through uint32_t before widening, or a set bit 31
// of the low half would sign-extend into the high half.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ u32x4 buffer_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

__device__ __forceinline__ uint16_t buffer_load_b16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane l's
// bytes land at lds + 16*l; `lds` must be the same for the whole wave.  Out-of-range lanes
// read zeros like any buffer load.
__device__ __forceinline__ void buffer_load_lds_b128(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): inside each group of 16 lanes, lane t receives
// element t % 4 of the 8-byte rows addressed by lanes t/4, t/4 + 4, t/4 + 8 and t/4 + 12.
__device__ __forceinline__ u32x2 lds_read_tr16_b64(const void* lds) {
    typedef short short4_v __attribute__((__vector_size__(4 * sizeof(short))));
    const auto pa = (__attribute__((address_space(3))) short4_v*)(const_cast<void*>(lds));
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(pa));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// Two floats -> two bf16 (round to nearest even) packed in one dword (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (lane ^ 32).  v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second; with both operands equal, a lane of the
// lower half finds its partner's value in the second result and a lane of the upper half in
// the first.
__device__ __forceinline__ float swap_halves(float x) {
    const int xi = __builtin_bit_cast(int, x);
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// max(x of this lane, x of lane ^ 32, y).  v_permlane32_swap on two copies of x leaves the lower
// half's x in one register and the upper half's in the other on every lane, so one v_max3 takes
// the maximum without a lane select.  Written as one asm block: the builtin's second result is
// miscompiled by this compiler when it is not consumed through a lane select.  The s_nop 1 gives
// the two wait states a VALU write needs before v_permlane32_swap reads it.  The compiler adds no
// wait states before inline asm for other producers: x and y must not come straight from an MFMA.
__device__ __forceinline__ float max_with_partner(float x, float y) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_max3_f32 %0, %0, %1, %2"
                 : "+v"(a), "+v"(b)
                 : "v"(y));
    return a;
}

// The O^T accumulators of one lane (one output row; in each 8-channel group the lane holds 4
// channels and lane ^ 32 the other 4), scaled by inv and rounded to bf16, stored to that row:
// lanes l and l + 32 trade one 4-channel half per pair of groups, so that every lane stores 16
// contiguous bytes (half the store instructions of 8-byte pieces).  Both lanes of a pair must
// be active.
template <int CBLK>
__device__ __forceinline__ void store_o_row(uint16_t* orow, const f32x16 (&oacc)[CBLK], float inv, int half) {
    auto swp = [](uint32_t x) __attribute__((always_inline)) {
        return __builtin_bit_cast(uint32_t, swap_halves(__builtin_bit_cast(float, x)));
    };
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
            uint32_t w[2][2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int grp = 2 * gp + k;
                w[k][0] = pack_bf16x2(oacc[cb][grp * 4 + 0] * inv, oacc[cb][grp * 4 + 1] * inv);
                w[k][1] = pack_bf16x2(oacc[cb][grp * 4 + 2] * inv, oacc[cb][grp * 4 + 3] * inv);
            }
            // half 0 keeps group 2gp and takes its partner's half of it; half 1 keeps 2gp + 1
            const uint32_t r0 = swp(half ? w[0][0] : w[1][0]);
            const uint32_t r1 = swp(half ? w[0][1] : w[1][1]);
            const int ch = cb * 32 + (2 * gp + half) * 8;
            *reinterpret_cast<u32x4*>(orow + ch) =
                half ? u32x4{r0, r1, w[1][0], w[1][1]} : u32x4{w[0][0], w[0][1], r0, r1};
        }
    }
}

__device__ __forceinline__ float max3(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

// acc + lo + hi of a packed pair of bf16 values (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

}  // namespace mha
