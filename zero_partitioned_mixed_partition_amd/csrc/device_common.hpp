// Device helpers shared by the gfx950 kernels: bf16 conversion, 16-byte
// streaming loads/stores, and fixed-order fp64 block reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace zero {
namespace dev {

constexpr int kWave = 64;   // CDNA wavefront width

// Native 16-byte vectors (8 bf16 or 4 fp32 lanes); loads and stores of these
// become single dwordx4 memory instructions.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN with the quiet bit
// set (sign and top payload bits kept); overflow rounds to infinity.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x0040u;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet : rounded;
}

// Low and high bf16 of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Streaming (non-temporal) 16-byte accesses: every byte is touched once per
// step, so nothing is worth keeping in the caches.
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
    return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_stream(T* p, const T& v) {
    __builtin_nontemporal_store(v, p);
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
