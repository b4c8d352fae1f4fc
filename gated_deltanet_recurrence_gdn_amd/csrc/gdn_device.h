// gdn_device.h -- small gfx950 device helpers used by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8), and
// each XCD has its own L2.  This bijection gives every XCD a contiguous range
// of logical block ids, so neighbouring logical blocks (which read the same
// q/k rows) share an L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int xcd = bid % kXcd, idx = bid / kXcd;
    const int base = nblocks / kXcd, rem = nblocks % kXcd;
    return xcd * base + (xcd < rem ? xcd : rem) + idx;
}

// DPP lane exchange inside a 16-lane row (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes (LPR = 4, 8 or 16); every lane of a
// group receives the group's sum.  quad_perm [1,0,3,2] and [2,3,0,1] make the
// quad sums; row_half_mirror then pairs the two quads of each 8 lanes, and
// row_mirror the two halves of each 16 lanes.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "group of 4, 8 or 16 lanes");
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    if constexpr (LPR >= 8) x += dpp_f32<0x141>(x);
    if constexpr (LPR >= 16) x += dpp_f32<0x140>(x);
    return x;
}

// Two sums over the same lane groups, step by step: each DPP step of one sum
// fills the other's data-hazard slot, so neither needs wait states.
template <int LPR>
__device__ __forceinline__ void group_sum2(float& x, float& y) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "group of 4, 8 or 16 lanes");
    x += dpp_f32<0xB1>(x);
    y += dpp_f32<0xB1>(y);
    x += dpp_f32<0x4E>(x);
    y += dpp_f32<0x4E>(y);
    if constexpr (LPR >= 8) {
        x += dpp_f32<0x141>(x);
        y += dpp_f32<0x141>(y);
    }
    if constexpr (LPR >= 16) {
        x += dpp_f32<0x140>(x);
        y += dpp_f32<0x140>(y);
    }
}

// Makes each of EPL fp32 values an opaque register value (an empty asm that
// "modifies" them in place, so nothing is copied).  A conversion of such a
// value to f16 then rounds the given fp32 number, two per v_cvt_pk_f16_f32,
// instead of the compiler refolding the producing multiply-add into a
// mixed-precision one (one instruction per element).
template <int EPL>
__device__ __forceinline__ void opaque_f32x8(float (&x)[EPL]) {
#pragma unroll
    for (int j = 0; j < EPL; j += 8)
        asm volatile("" : "+v"(x[j]), "+v"(x[j + 1]), "+v"(x[j + 2]), "+v"(x[j + 3]), "+v"(x[j + 4]), "+v"(x[j + 5]),
                     "+v"(x[j + 6]), "+v"(x[j + 7]));
}

// Eight fp32 values -> f16, round to nearest even, two per instruction.
__device__ __forceinline__ f16x8 to_f16x8(float x0, float x1, float x2, float x3, float x4, float x5, float x6,
                                          float x7) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 a = __builtin_convertvector(f2{x0, x1}, h2), b = __builtin_convertvector(f2{x2, x3}, h2);
    const h2 c = __builtin_convertvector(f2{x4, x5}, h2), d = __builtin_convertvector(f2{x6, x7}, h2);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// bf16 <-> fp32.  bf16 widening is exact; narrowing is the hardware's
// v_cvt_pk_bf16_f32 (round to nearest even, NaN stays NaN), with no branch.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Load 8 consecutive elements (bf16 or fp32) as fp32.
__device__ __forceinline__ void load8_as_f32(const void* base, size_t idx, bool bf16, float (&x)[8]) {
    if (bf16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        const float* p = static_cast<const float*>(base) + idx;
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
}

__device__ __forceinline__ float load1_as_f32(const void* base, size_t idx, bool bf16) {
    if (bf16) return __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(base)[idx] << 16);
    return static_cast<const float*>(base)[idx];
}

// Store of write-once data: non-temporal when NT (small launches, where it
// shortens the end-of-kernel drain), plain otherwise (large streaming launches,
// where plain stores measured faster).  A compile-time choice: with a runtime
// branch the compiler merges both stores and drops the non-temporal hint.
template <bool NT, typename T>
__device__ __forceinline__ void store_stream(T v, T* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

__device__ __forceinline__ void store_out(void* out, size_t idx, float o, int dtype) {
    if (dtype == 0) static_cast<float*>(out)[idx] = o;
    else if (dtype == 2) static_cast<_Float16*>(out)[idx] = (_Float16)o;
    else static_cast<uint16_t*>(out)[idx] = f32_to_bf16(o);
}

}  // namespace gdn
