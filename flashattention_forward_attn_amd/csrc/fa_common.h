// fa_common.h -- types and small device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Combine the two lane halves (lanes i and i ^ 32) with one v_permlane32_swap:
// afterwards {a, b} of every lane hold x from lane i % 32 and lane i % 32 + 32.
__device__ __forceinline__ float halves_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Make the compiler treat v as produced here: values loaded once before a loop
// then carry no memory-counter dependency into it.
template <typename T>
__device__ __forceinline__ void launder(T& v) {
    asm volatile("" : "+v"(v));
}

__device__ __forceinline__ float wave_max(float x) {
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
    for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, kWave));
    return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
    for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off, kWave));
    return x;
}

// Pack two fp32 values into bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 p;
    p[0] = (bf16)lo;
    p[1] = (bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

// The score sign applied to a 32-bit word of the register-resident score operand
// (and_mask zeroes it for a zero scale, xor_mask flips sign bits for a negative one).
__device__ __forceinline__ uint32_t score_signed(uint32_t w, uint32_t and_mask, uint32_t xor_mask) {
    return (w & and_mask) ^ xor_mask;
}

// Number of keys row `q` may attend to: keys j < limit are candidates, then the
// causal condition j <= q is applied on top (limit <= q + 1).
__device__ __forceinline__ int row_key_limit(int q, int N, bool causal, const int32_t* kv_limit_row) {
    if (q >= N) return 0;
    int lim = N;
    if (kv_limit_row) {
        int v = *kv_limit_row;
        v = v < 0 ? 0 : v;
        lim = v < lim ? v : lim;
    }
    if (causal && q + 1 < lim) lim = q + 1;
    return lim;
}

}  // namespace fa
