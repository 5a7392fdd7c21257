// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// 2^x on the transcendental unit (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Full 64-lane butterfly reductions.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap): the two
// halves of a 32x32 MFMA accumulator column hold the same query row.
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transpose 4 keys x 4 dims of bf16 (rows[j] = dims d..d+3 of key j, as two
// bf16 pairs) into 4 dims x 4 keys: out[i] = keys 0..3 of dim d+i, as two
// bf16 pairs, ready for one 8-byte LDS store per dim.
__device__ __forceinline__ void transpose4x4_bf16(const u32x2 rows[4], u32x2 out[4]) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
        const uint32_t a0 = rows[0][half], a1 = rows[1][half];
        const uint32_t a2 = rows[2][half], a3 = rows[3][half];
        out[2 * half] = u32x2{__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                              __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
        out[2 * half + 1] = u32x2{__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                                  __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
    }
}

// Checked build (compiled with ATTN_CHECKED=1): the kernels validate the
// device-side indices they are given, record what was out of range in a
// per-device error word and go on with a safe value, so a bad block table or
// length cannot make them read outside the page pool.  The release build
// compiles these checks away.
#ifndef ATTN_CHECKED
#define ATTN_CHECKED 0
#endif
constexpr unsigned kDevErrKvLen = 1u;   // a length outside [0, its host bound]
constexpr unsigned kDevErrPage = 2u;    // a page index outside [0, num_pages)

// Flags a length outside [0, bound]; the caller clamps it as in the release
// build.
__device__ __forceinline__ void check_len(int len, int bound, unsigned* err) {
    if constexpr (ATTN_CHECKED) {
        if ((len < 0 || len > bound) && err) atomicOr(err, kDevErrKvLen);
    }
}
// A page index, or page 0 (inside any non-empty pool) with the error flagged
// when it lies outside [0, num_pages).
__device__ __forceinline__ int checked_page(int p, int num_pages, unsigned* err) {
    if constexpr (ATTN_CHECKED) {
        if (p < 0 || p >= num_pages) {
            if (err) atomicOr(err, kDevErrPage);
            return 0;
        }
    }
    return p;
}

}  // namespace attn
