// Device helpers shared by the gfx950 kernels: bf16 conversion, 16-byte
// streaming loads/stores, and fixed-order fp64 block reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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

// Streaming accesses: every byte is touched once per step, so nothing is worth
// keeping in the caches. Loads are non-temporal.
//
// Stores write through to memory: a buffer store carrying the device-scope
// (sc1) and non-temporal (nt) cache bits, where a plain non-temporal store
// leaves dirty lines in the XCD's L2 to be written back later. Measured on
// MI355X: AdamW 66.6 us against 69.3 us at 15.6 M elements, 528 us against
// 540 us at 125 M; a 16-byte-per-lane copy of 2.6 GB 786-789 us against
// 809-812 us. Cache bits on the loads measured no difference.
//
// A buffer store addresses memory as a 64-bit base, which must be the same
// for every lane of the wave, plus a 32-bit offset per lane. Three forms:
//
//   st_stream(p, v)          the base is the first active lane's address less
//                            2 GiB, each lane's offset its distance from that
//                            base. Contract: every active lane stores within
//                            2 GiB of the first active lane's address. Used by
//                            kernels whose waves store one contiguous run of at
//                            most 64 accesses (AdamW, the reduce, the copy of
//                            one piece, the gather into one tensor).
//   st_stream_at(b, off, v)  the caller passes the base b, the same pointer in
//                            every lane, and each lane's byte offset off from it
//                            (below 2^32). For waves that store into several
//                            buffers far apart (the Shard(0) flatten into two
//                            ranks' buffers): one call per buffer, each with
//                            that buffer's base.
//   st_stream_any(p, v)      a global non-temporal store: any address.
//
// The record count of the buffer is the full 32-bit range, so the buffer's own
// range check never drops a store (bounds are the callers', as with a global
// store).
#ifndef ZERO_NT_LOADS
#define ZERO_NT_LOADS 1
#endif
// 1: write-through buffer stores (sc1 nt); 0: global non-temporal stores.
#ifndef ZERO_THROUGH_STORES
#define ZERO_THROUGH_STORES 1
#endif
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
#if ZERO_NT_LOADS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

constexpr int kRawBufferWord3 = 0x00020000;   // untyped buffer, 32-bit data format
constexpr int kThroughCpol = 0x12;            // sc1 (device scope) | nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t through_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, kRawBufferWord3);
}

// The first active lane's address less 2 GiB (or 0), as the wave's base; `off`
// receives this lane's distance from it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t through_base(const void* p, uint32_t& off) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    const uint64_t first = (static_cast<uint64_t>(hi) << 32) | lo;
    const uint64_t base = first >= (uint64_t(1) << 31) ? first - (uint64_t(1) << 31) : 0;
    off = static_cast<uint32_t>(a - base);
    return through_rsrc(reinterpret_cast<const void*>(base));
}

__device__ __forceinline__ void through_store(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kThroughCpol);
}
__device__ __forceinline__ void through_store(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kThroughCpol);
}
__device__ __forceinline__ void through_store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    through_store(r, off, __builtin_bit_cast(uint32_t, v));
}
__device__ __forceinline__ void through_store(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kThroughCpol);
}
__device__ __forceinline__ void through_store(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kThroughCpol);
}
template <typename T>
__device__ __forceinline__ void through_store(__amdgpu_buffer_rsrc_t r, uint32_t off, const T& v) {
    static_assert(sizeof(T) == 8 || sizeof(T) == 16, "8- or 16-byte vector");
    typedef typename std::conditional<sizeof(T) == 8, u32x2, u32x4>::type W;
    through_store(r, off, __builtin_bit_cast(W, v));
}

template <typename T>
__device__ __forceinline__ void st_stream(T* p, const T& v) {
#if ZERO_THROUGH_STORES
    uint32_t off;
    const __amdgpu_buffer_rsrc_t r = through_base(p, off);
    through_store(r, off, v);
#else
    __builtin_nontemporal_store(v, p);
#endif
}

template <typename T>
__device__ __forceinline__ void st_stream_at(const void* base, uint32_t off, const T& v) {
#if ZERO_THROUGH_STORES
    through_store(through_rsrc(base), off, v);
#else
    __builtin_nontemporal_store(v, reinterpret_cast<T*>(static_cast<char*>(const_cast<void*>(base)) + off));
#endif
}

template <typename T>
__device__ __forceinline__ void st_stream_any(T* p, const T& v) {
    __builtin_nontemporal_store(v, p);
}

// Loads through a wave-uniform base (the counterpart of st_stream_at): `base`
// the same in every lane, `off` the lane's byte offset from it (below 2^32);
// non-temporal as ld_stream.
#if ZERO_NT_LOADS
constexpr int kLoadCpol = 0x2;                // nt
#else
constexpr int kLoadCpol = 0;
#endif
__device__ __forceinline__ uint32_t ld_stream_at_b32(const void* base, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(through_rsrc(base), off, 0, kLoadCpol);
}
__device__ __forceinline__ uint16_t ld_stream_at_b16(const void* base, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(through_rsrc(base), off, 0, kLoadCpol);
}

// The first active lane's value of a 64-bit quantity (wave-uniform).
__device__ __forceinline__ int64_t first_lane(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Entry of workgroup blockIdx.x in a launch's XCD-major table index (the
// layout is described with xcd_major_index on the host side).
__device__ __forceinline__ int64_t xcd_major_entry(int64_t blk0, int64_t per) {
    const int64_t x = blockIdx.x;
    return blk0 + (x & 7) * per + (x >> 3);
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

// Visits R replicas' V-sized values at index i (V units past p[k] + src_off),
// in replica order, with B loads in flight: each batch's loads are issued
// together, unconditionally, before the first value is used. A batch of fewer
// than B replicas (the last R mod B) loads the batch's first replica in place
// of the missing ones and does not visit those copies. (A guarded load per
// replica becomes a branch per load, and the compiler then waits for each load
// before issuing the next: measured on MI355X, the one-pass reduce and AdamW
// over 8 replicas of a 164 M-element shard ran at 46% of HBM peak that way
// and at 81% with this form.) `p` is indexed with wave-uniform values only.
template <int B, typename V, typename Visit>
__device__ __forceinline__ void for_replicas(const uint16_t* const* p, int n_rep, int64_t src_off,
                                             int64_t i, Visit visit) {
    int k0 = 0;
    for (; k0 + B <= n_rep; k0 += B) {
        V x[B];
#pragma unroll
        for (int k = 0; k < B; ++k) x[k] = ld_stream(reinterpret_cast<const V*>(p[k0 + k] + src_off) + i);
#pragma unroll
        for (int k = 0; k < B; ++k) visit(x[k]);
    }
    const int kn = n_rep - k0;
    if (kn > 0) {
        V x[B];
#pragma unroll
        for (int k = 0; k < B; ++k)
            x[k] = ld_stream(reinterpret_cast<const V*>(p[k0 + (k < kn ? k : 0)] + src_off) + i);
#pragma unroll
        for (int k = 0; k < B; ++k)
            if (k < kn) visit(x[k]);
    }
}

}  // namespace dev
}  // namespace zero
