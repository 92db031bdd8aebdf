// Device helpers shared by the gfx950 kernels: bf16 conversion, 16-byte
// streaming loads/stores, and fixed-order fp64 block reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace zero {
namespace dev {

constexpr int kWave = 64;   // CDNA wavefront width

// Native vectors; loads and stores of these become single dwordx4 / dwordx2
// memory instructions.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Low and high bf16 of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two bf16 in one 32-bit word (lo in the low half). gfx950's
// v_cvt_pk_bf16_f32 rounds to nearest even, keeps subnormals, sends overflow
// to infinity and returns a NaN input as that NaN with the quiet bit set
// (sign and top payload bits kept): the same bits as the integer formula
// (u + 0x7FFF + ((u >> 16) & 1)) >> 16 for non-NaN u, and (u >> 16) | 0x40
// for NaN, which a GPU test checks over every rounding case.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const bf16x2 r = __builtin_convertvector((f32x2{lo, hi}), bf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &r, sizeof(u));
    return u;
}

__device__ __forceinline__ uint32_t f32_to_bf16(float x) { return pack_bf16(x, x) & 0xFFFFu; }

// Streaming (non-temporal) 16-byte accesses: every byte is touched once per
// step, so nothing is worth keeping in the caches.
#ifndef ZERO_NT_LOADS
#define ZERO_NT_LOADS 1
#endif
#ifndef ZERO_NT_STORES
#define ZERO_NT_STORES 1
#endif
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
#if ZERO_NT_LOADS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
template <typename T>
__device__ __forceinline__ void st_stream(T* p, const T& v) {
#if ZERO_NT_STORES
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Sum of one double per thread over a block of kThreads threads, in a fixed
// order (butterfly inside each wave, then waves in index order). The result
// is valid in thread 0. `lds` holds kThreads / kWave doubles.
template <int kThreads>
__device__ __forceinline__ double block_sum(double x, double* lds) {
    static_assert(kThreads % kWave == 0, "whole waves");
    constexpr int kWaves = kThreads / kWave;
    x = wave_sum(x);
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    if (lane == 0) lds[wave] = x;
    __syncthreads();
    double total = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += lds[w];
    }
    return total;
}

}  // namespace dev
}  // namespace zero
