// Shard-local gradient reduction, squared-norm partials and the clip
// coefficient (gfx950).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "Execution Flow for ZeRO-1", step 2:
// each rank receives the gradient of its own partition averaged over the
// ranks; section "ZeRO-Stage 2": the reduction happens bucket by bucket. The
// kernel here is the receiving rank's arithmetic: R replica buffers in HBM,
// summed in replica order in fp32, divided by R, rounded once to bf16.
//
// Memory: per shard element R bf16 reads and one bf16 write, (2R + 2) bytes.
// Each thread handles 8 elements per 16-byte access and takes the replicas in
// batches of 8, adding them in order into its accumulators (the guarded load
// per replica compiles to one load in flight at a time, which measured faster
// here than issuing a batch at once); the grid is capped and threads stride. Large windows of at most 8 replicas,
// given a workspace for a partial per workgroup, take a one-pass form instead
// (a lane per element pair, the grid covering the window once); so does the
// standalone squared norm on large inputs. Both sum the partials in two
// fixed-order levels.
//
// The squared norm (not on the pages; needed by the global-norm clip) sums
// exact fp64 squares of bf16 values: per-thread fp64 partials, a butterfly in
// each wavefront, waves in order through LDS, one partial per workgroup in the
// caller's workspace, then one or two fixed-order passes add the workgroup
// partials. No floating-point atomics, and a grid that depends only on n and on
// which form the workspace allows: results repeat bit for bit, on any device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "device_common.hpp"
#include "internal.hpp"
#include "pieces.hpp"

#pragma clang fp contract(off)

namespace {

using zero::dev::u32x4;

constexpr int kThreads = 256;
// Grid caps (measured on MI355X: the replica reduce keeps more bytes in flight
// per lane and does best with fewer, longer-lived workgroups than the one-read
// squared norm), and so the number of workgroup partials the workspace holds.
// Below the cap each thread handles one group of 8 elements; above it threads
// stride.
// The grid depends on n only, so the summation order (and the fp64 result)
// is the same on every device. Re-measured for the replica reduce, two runs,
// with its final sum: caps of 512, 1,024, 2,048 and 4,096 workgroups took
// 4,453, 2,823-2,824, 2,522-2,523 and 2,513-2,516 us on Llama-3-8B (64
// replicas) and 80.2-80.3, 53.3-53.4, 47.0 and 47.5 us on GPT-2 (8).
#ifndef ZERO_REDUCE_MAX_BLOCKS
#define ZERO_REDUCE_MAX_BLOCKS 2048
#endif
#ifndef ZERO_SQNORM_MAX_BLOCKS
#define ZERO_SQNORM_MAX_BLOCKS 4096
#endif
constexpr int kMaxPartials = ZERO_REDUCE_MAX_BLOCKS > ZERO_SQNORM_MAX_BLOCKS
                                 ? ZERO_REDUCE_MAX_BLOCKS : ZERO_SQNORM_MAX_BLOCKS;
#ifndef ZERO_REDUCE_BATCH
#define ZERO_REDUCE_BATCH 8
#endif
constexpr int kReplicaBatch = ZERO_REDUCE_BATCH;   // replicas per load batch
// 1: the grid-stride kernel's replica loads through zero::dev::for_replicas
// (each batch issued at once, the adds after). 0 (default): a guarded load per
// replica, which the compiler issues one at a time. Measured on MI355X, 64
// replicas over six 25 M-element buckets of a 125 M-element shard: 2.586 ms
// with one load in flight, 2.85 ms with batches of 8 (3.24 ms with batches of
// 1 through the helper); no difference at 8 replicas.
#ifndef ZERO_REDUCE_BATCHED_ISSUE
#define ZERO_REDUCE_BATCHED_ISSUE 0
#endif

// 1: the reduce kernels store the averaged gradient with plain (cache-allocating)
// stores, so a following AdamW can read it from cache; 0 (default): streaming
// write-through stores. Measured on MI355X, three runs: the reduce 7% slower
// on GPT-2 (51.2-51.8 against 47.6-47.9 us), 5% on Llama-3-8B, 4% on the 1.3B
// GPT; AdamW after it 1.5% faster on Llama-3-8B only; steps level or slower.
#ifndef ZERO_REDUCE_OUT_CACHED
#define ZERO_REDUCE_OUT_CACHED 0
#endif
template <typename V>
__device__ __forceinline__ void store_grad(V* p, const V& v) {
#if ZERO_REDUCE_OUT_CACHED
    *p = v;
#else
    zero::dev::st_stream(p, v);
#endif
}

struct ReplicaTable {
    const uint16_t* p[ZERO_MAX_REPLICAS];
};

__device__ __forceinline__ double sq8(const u32x4& w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double a = static_cast<double>(zero::dev::lo_bf16(ws[j]));
        const double b = static_cast<double>(zero::dev::hi_bf16(ws[j]));
        s += a * a;
        s += b * b;
    }
    return s;
}

__device__ __forceinline__ double sq1(uint16_t h) {
    const double a = static_cast<double>(zero::dev::bf16_to_f32(h));
    return a * a;
}

__device__ __forceinline__ void store_partial(double sq, double* partials) {
    __shared__ double lds[kThreads / zero::dev::kWave];
    const double total = zero::dev::block_sum<kThreads>(sq, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

#ifndef ZERO_REDUCE_EPT
#define ZERO_REDUCE_EPT 8
#endif
constexpr int kEpt = ZERO_REDUCE_EPT;   // elements per lane per replica access

template <int E> struct Bits;           // E bf16 values in one access
template <> struct Bits<8> { typedef u32x4 T; };
template <> struct Bits<4> { typedef zero::dev::u32x2 T; };
template <> struct Bits<2> { typedef uint32_t T; };

[[maybe_unused]] __device__ __forceinline__ uint32_t word(uint32_t x, int) { return x; }
[[maybe_unused]] __device__ __forceinline__ uint32_t word(const zero::dev::u32x2& x, int j) { return x[j]; }
[[maybe_unused]] __device__ __forceinline__ uint32_t word(const u32x4& x, int j) { return x[j]; }
[[maybe_unused]] __device__ __forceinline__ void set_word(uint32_t& x, int, uint32_t w) { x = w; }
[[maybe_unused]] __device__ __forceinline__ void set_word(zero::dev::u32x2& x, int j, uint32_t w) { x[j] = w; }
[[maybe_unused]] __device__ __forceinline__ void set_word(u32x4& x, int j, uint32_t w) { x[j] = w; }

// Vector path. src_off: element offset into each replica buffer of the first
// element to reduce; out: first output element; n: elements to reduce. The
// caller guarantees every replica + src_off and out are aligned to E elements.
// kGroups: groups per pass when the replicas fit one load batch. A lane then
// issues the loads of kGroups groups (kGroups * R accesses in flight) before
// it adds them; each lane still adds its groups to the fp64 norm in index
// order, so every variant gives the same bits. A separate kernel per value,
// so the one-group form keeps its lower register count and occupancy.
// Measured on MI355X with 8 replicas: 2 groups +4.5% at 164 M elements,
// -2% at 15.6 M; with 64 replicas the wider form would cost 13%.
#ifndef ZERO_REDUCE_TWO_GROUPS_FROM
#define ZERO_REDUCE_TWO_GROUPS_FROM (int64_t(1) << 26)
#endif
constexpr int64_t kTwoGroupsFrom = ZERO_REDUCE_TWO_GROUPS_FROM;   // shard elements
// Windows from this many elements take the one-pass kernel (reduce_pass), when
// the caller's workspace holds its partials (zero_reduce_workspace_bytes).
#ifndef ZERO_REDUCE_ONE_PASS_FROM
#define ZERO_REDUCE_ONE_PASS_FROM (int64_t(1) << 24)
#endif
constexpr int64_t kOnePassFrom = ZERO_REDUCE_ONE_PASS_FROM;

template <bool kNorm, int kGroups>
__global__ __launch_bounds__(kThreads) void reduce_vec(ReplicaTable reps, int n_rep,
                                                       int64_t src_off,
                                                       uint16_t* __restrict__ out, int64_t n,
                                                       double* __restrict__ partials) {
    typedef typename Bits<kEpt>::T V;
    constexpr int kWords = kEpt / 2;
    const float r = static_cast<float>(n_rep);
    const int64_t groups = n / kEpt;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    double sq = 0.0;
    auto finish_group = [&](int64_t i, const float* acc) {
        V o;
        uint32_t ow[kWords];
#pragma unroll
        for (int j = 0; j < kWords; ++j) {
            ow[j] = zero::dev::pack_bf16(acc[2 * j] / r, acc[2 * j + 1] / r);
            if (kNorm) {
                const double a = static_cast<double>(zero::dev::lo_bf16(ow[j]));
                const double b = static_cast<double>(zero::dev::hi_bf16(ow[j]));
                sq += a * a;
                sq += b * b;
            }
        }
#pragma unroll
        for (int j = 0; j < kWords; ++j) set_word(o, j, ow[j]);
        store_grad(reinterpret_cast<V*>(out) + i, o);
    };
    if (kGroups > 1 && n_rep <= kReplicaBatch) {
        for (int64_t i0 = tid; i0 < groups; i0 += kGroups * stride) {
            V x[kGroups][kReplicaBatch];
#pragma unroll
            for (int q = 0; q < kGroups; ++q) {
                const int64_t i = i0 + q * stride;
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k)
                    if (k < n_rep && i < groups)
                        x[q][k] = zero::dev::ld_stream(reinterpret_cast<const V*>(reps.p[k] + src_off) + i);
            }
#pragma unroll
            for (int q = 0; q < kGroups; ++q) {
                const int64_t i = i0 + q * stride;
                if (i >= groups) break;
                float acc[kEpt];
#pragma unroll
                for (int j = 0; j < kEpt; ++j) acc[j] = 0.0f;
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k) {
                    if (k < n_rep) {
#pragma unroll
                        for (int j = 0; j < kWords; ++j) {
                            const uint32_t w = word(x[q][k], j);
                            acc[2 * j] = acc[2 * j] + zero::dev::lo_bf16(w);
                            acc[2 * j + 1] = acc[2 * j + 1] + zero::dev::hi_bf16(w);
                        }
                    }
                }
                finish_group(i, acc);
            }
        }
    } else {
        for (int64_t i = tid; i < groups; i += stride) {
            float acc[kEpt];
#pragma unroll
            for (int j = 0; j < kEpt; ++j) acc[j] = 0.0f;
#if ZERO_REDUCE_BATCHED_ISSUE
            zero::dev::for_replicas<kReplicaBatch, V>(reps.p, n_rep, src_off, i, [&](const V& x) {
#pragma unroll
                for (int j = 0; j < kWords; ++j) {
                    const uint32_t w = word(x, j);
                    acc[2 * j] = acc[2 * j] + zero::dev::lo_bf16(w);
                    acc[2 * j + 1] = acc[2 * j + 1] + zero::dev::hi_bf16(w);
                }
            });
#else
            for (int k0 = 0; k0 < n_rep; k0 += kReplicaBatch) {
                V x[kReplicaBatch];
                const int kn = n_rep - k0 < kReplicaBatch ? n_rep - k0 : kReplicaBatch;
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k)
                    if (k < kn)
                        x[k] = zero::dev::ld_stream(reinterpret_cast<const V*>(reps.p[k0 + k] + src_off) + i);
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k) {
                    if (k < kn) {
#pragma unroll
                        for (int j = 0; j < kWords; ++j) {
                            const uint32_t w = word(x[k], j);
                            acc[2 * j] = acc[2 * j] + zero::dev::lo_bf16(w);
                            acc[2 * j + 1] = acc[2 * j + 1] + zero::dev::hi_bf16(w);
                        }
                    }
                }
            }
#endif
            finish_group(i, acc);
        }
    }
    // Ragged tail (< E elements), one per thread of the first threads.
    const int64_t tail = n - groups * kEpt;
    if (tid < tail) {
        const int64_t e = groups * kEpt + tid;
        float acc = 0.0f;
        for (int k = 0; k < n_rep; ++k) acc = acc + zero::dev::bf16_to_f32(reps.p[k][src_off + e]);
        const uint16_t h = static_cast<uint16_t>(zero::dev::f32_to_bf16(acc / r));
        out[e] = h;
        if (kNorm) sq += sq1(h);
    }
    if (kNorm) store_partial(sq, partials);
}

// Rows form of the vector path (ZERO_REDUCE_ROWS = G > 1; 1, the default,
// keeps reduce_vec): a workgroup covers G * kThreads consecutive 8-element
// groups per pass, lane l the groups base + l + q * kThreads (q < G). For each
// replica in order a lane issues its G loads together, so a workgroup's loads
// in flight all fall in one contiguous G * 4 KB run of one replica; then it
// adds them. Lanes past the end load the last group again (every load is
// unconditional) and drop it. Each element's sum is the same as reduce_vec's.
// Measured on MI355X, two runs, reduce phase with its final sum: Llama-3-8B
// (64 replicas, six 25 M buckets) 2,526-2,527 us with reduce_vec, 2,709-2,710
// with G = 2, 2,675 with 4, 2,571-2,578 with 8; GPT-2 (8 replicas) 47.5 us,
// 47.3-47.4, 48.4 and 47.9-48.1 us. More loads in flight per lane cost even
// when they all fall in one replica's run, so reduce_vec stays.
#ifndef ZERO_REDUCE_ROWS
#define ZERO_REDUCE_ROWS 1
#endif
constexpr int kRows = ZERO_REDUCE_ROWS;

template <bool kNorm>
__global__ __launch_bounds__(kThreads) void reduce_rows(ReplicaTable reps, int n_rep, int64_t src_off,
                                                        uint16_t* __restrict__ out, int64_t n,
                                                        double* __restrict__ partials) {
    static_assert(kEpt == 8, "the rows form takes 16-byte groups");
    const float r = static_cast<float>(n_rep);
    const int64_t groups = n / 8;
    const int64_t span = int64_t(kRows) * kThreads;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * span;
    double sq = 0.0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * span; base < groups; base += stride) {
        int64_t at[kRows];
#pragma unroll
        for (int q = 0; q < kRows; ++q) {
            const int64_t i = base + threadIdx.x + int64_t(q) * kThreads;
            at[q] = i < groups ? i : groups - 1;
        }
        float acc[kRows][8];
#pragma unroll
        for (int q = 0; q < kRows; ++q)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[q][j] = 0.0f;
        for (int k = 0; k < n_rep; ++k) {
            const u32x4* src = reinterpret_cast<const u32x4*>(reps.p[k] + src_off);
            u32x4 x[kRows];
#pragma unroll
            for (int q = 0; q < kRows; ++q) x[q] = zero::dev::ld_stream(src + at[q]);
#pragma unroll
            for (int q = 0; q < kRows; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[q][2 * j] = acc[q][2 * j] + zero::dev::lo_bf16(x[q][j]);
                    acc[q][2 * j + 1] = acc[q][2 * j + 1] + zero::dev::hi_bf16(x[q][j]);
                }
        }
#pragma unroll
        for (int q = 0; q < kRows; ++q) {
            const int64_t i = base + threadIdx.x + int64_t(q) * kThreads;
            if (i >= groups) break;
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = zero::dev::pack_bf16(acc[q][2 * j] / r, acc[q][2 * j + 1] / r);
            if (kNorm) sq += sq8(w);
            store_grad(reinterpret_cast<u32x4*>(out) + i, w);
        }
    }
    // Ragged tail (< 8 elements), one per thread of the first threads.
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t tail = n - groups * 8;
    if (tid < tail) {
        const int64_t e = groups * 8 + tid;
        float acc = 0.0f;
        for (int k = 0; k < n_rep; ++k) acc = acc + zero::dev::bf16_to_f32(reps.p[k][src_off + e]);
        const uint16_t h = static_cast<uint16_t>(zero::dev::f32_to_bf16(acc / r));
        out[e] = h;
        if (kNorm) sq += sq1(h);
    }
    if (kNorm) store_partial(sq, partials);
}

// Any alignment: one element per thread.
template <bool kNorm>
__global__ __launch_bounds__(kThreads) void reduce_scalar(ReplicaTable reps, int n_rep,
                                                          int64_t src_off,
                                                          uint16_t* __restrict__ out, int64_t n,
                                                          double* __restrict__ partials) {
    const float r = static_cast<float>(n_rep);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    double sq = 0.0;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; e < n; e += stride) {
        float acc = 0.0f;
        for (int k = 0; k < n_rep; ++k) acc = acc + zero::dev::bf16_to_f32(reps.p[k][src_off + e]);
        const uint16_t h = static_cast<uint16_t>(zero::dev::f32_to_bf16(acc / r));
        out[e] = h;
        if (kNorm) sq += sq1(h);
    }
    if (kNorm) store_partial(sq, partials);
}

// One-pass form for large windows: each lane reduces W 32-bit words (2W
// elements), one access per replica, and the grid covers the window once, so
// workgroups retire in dispatch order and the chip works on a narrow sliding
// window of every replica. Measured on MI355X with 8 replicas over the 1.3 B
// GPT's 164 M-element shards (W = 1): 3.79 ms against 4.11 ms for the
// grid-stride kernel over all 8 ranks; below 2^24 elements the grid-stride
// kernel is faster (the GPT-2 shard: 48.7 against 51.1-51.8 us). Same
// per-element arithmetic as reduce_vec (replica order, one division, one
// rounding), so the same bits. Workgroup b = block0 + blockIdx.x reduces
// units [b * kThreads * kPassQ, (b + 1) * kThreads * kPassQ) of 2W elements,
// each lane kPassQ units kThreads apart (one contiguous run per workgroup); a
// ragged end is reduced element by element. The workgroup's squared-norm
// partial goes to partials[blockIdx.x].
// Units per lane, kThreads units apart. Measured on the 1.3 B GPT's shards
// (8 replicas): 1 unit 3.70 ms over all 8 ranks, 2 units 3.81, 4 units 4.02.
#ifndef ZERO_REDUCE_PASS_Q
#define ZERO_REDUCE_PASS_Q 1
#endif
constexpr int kPassQ = ZERO_REDUCE_PASS_Q;

template <bool kNorm, int W>
__global__ __launch_bounds__(kThreads) void reduce_pass(ReplicaTable reps, int n_rep,
                                                        int64_t src_off,
                                                        uint16_t* __restrict__ out, int64_t n,
                                                        int64_t block0,
                                                        double* __restrict__ partials) {
    typedef typename Bits<2 * W>::T V;
    constexpr int64_t E = 2 * W;
    const float r = static_cast<float>(n_rep);
    const int64_t base = (block0 + static_cast<int64_t>(blockIdx.x)) * kThreads * kPassQ;
    double sq = 0.0;
#pragma unroll
    for (int q = 0; q < kPassQ; ++q) {
        const int64_t i = base + int64_t(q) * kThreads + threadIdx.x;
        if (E * i + E <= n) {
            float acc[E];
#pragma unroll
            for (int j = 0; j < E; ++j) acc[j] = 0.0f;
            for (int k0 = 0; k0 < n_rep; k0 += kReplicaBatch) {
                V x[kReplicaBatch];
                const int kn = n_rep - k0 < kReplicaBatch ? n_rep - k0 : kReplicaBatch;
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k)
                    if (k < kn)
                        x[k] = zero::dev::ld_stream(reinterpret_cast<const V*>(reps.p[k0 + k] + src_off) + i);
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k) {
                    if (k < kn) {
#pragma unroll
                        for (int j = 0; j < W; ++j) {
                            const uint32_t w = word(x[k], j);
                            acc[2 * j] = acc[2 * j] + zero::dev::lo_bf16(w);
                            acc[2 * j + 1] = acc[2 * j + 1] + zero::dev::hi_bf16(w);
                        }
                    }
                }
            }
            V o;
#pragma unroll
            for (int j = 0; j < W; ++j) {
                const uint32_t ow = zero::dev::pack_bf16(acc[2 * j] / r, acc[2 * j + 1] / r);
                set_word(o, j, ow);
                if (kNorm) {
                    const double a = static_cast<double>(zero::dev::lo_bf16(ow));
                    const double b = static_cast<double>(zero::dev::hi_bf16(ow));
                    sq += a * a;
                    sq += b * b;
                }
            }
            store_grad(reinterpret_cast<V*>(out) + i, o);
        } else {                                      // ragged end: element by element
            for (int64_t e = E * i; e < n && e < E * i + E; ++e) {
                float acc = 0.0f;
                for (int k = 0; k < n_rep; ++k) acc = acc + zero::dev::bf16_to_f32(reps.p[k][src_off + e]);
                const uint16_t h = static_cast<uint16_t>(zero::dev::f32_to_bf16(acc / r));
                out[e] = h;
                if (kNorm) sq += sq1(h);
            }
        }
    }
    if (kNorm) store_partial(sq, partials);
}

__global__ __launch_bounds__(kThreads) void sqnorm_vec(const uint16_t* __restrict__ g, int64_t n,
                                                       double* __restrict__ partials) {
    const int64_t groups = n / 8;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    double sq = 0.0;
    for (int64_t i = tid; i < groups; i += stride)
        sq += sq8(zero::dev::ld_stream(reinterpret_cast<const u32x4*>(g) + i));
    const int64_t tail = n - groups * 8;
    if (tid < tail) sq += sq1(g[groups * 8 + tid]);
    store_partial(sq, partials);
}

// One-pass squared norm for large inputs: each lane reads kSqPassGroups
// groups of 8 values (16 bytes each, kThreads groups apart, so a workgroup
// reads one contiguous run); the grid covers the input once, a partial per
// workgroup (the reduce's one-pass reasoning: workgroups retire in dispatch
// order, a narrow sliding window). The n % 8 tail takes the slots just past
// the last group.
// 16-byte groups per lane (a workgroup reads 32 KB). Measured on MI355X over
// 2^30 values: 1 group 409-489 us, 4 groups 315-334, 8 groups 316-319 (84-85%
// of peak), 16 groups 331; the grid-stride kernel 360-365 us (74%).
#ifndef ZERO_SQNORM_PASS_GROUPS
#define ZERO_SQNORM_PASS_GROUPS 8
#endif
constexpr int kSqPassGroups = ZERO_SQNORM_PASS_GROUPS;

__global__ __launch_bounds__(kThreads) void sqnorm_pass(const uint16_t* __restrict__ g, int64_t n,
                                                        int64_t slot0,
                                                        double* __restrict__ partials) {
    // Workgroup b covers slots [(slot0 + b) * kThreads * Q, ... + kThreads * Q): slot s
    // is group s (s < n / 8) or tail element n/8*8 + (s - n/8).
    const int64_t groups = n / 8;
    const int64_t base = (slot0 + static_cast<int64_t>(blockIdx.x)) * kThreads * kSqPassGroups;
    u32x4 x[kSqPassGroups];
#pragma unroll
    for (int q = 0; q < kSqPassGroups; ++q) {
        const int64_t i = base + int64_t(q) * kThreads + threadIdx.x;
        if (i < groups) x[q] = zero::dev::ld_stream(reinterpret_cast<const u32x4*>(g) + i);
    }
    double sq = 0.0;
#pragma unroll
    for (int q = 0; q < kSqPassGroups; ++q) {
        const int64_t i = base + int64_t(q) * kThreads + threadIdx.x;
        if (i < groups) {
            sq += sq8(x[q]);
        } else {
            const int64_t e = groups * 8 + (i - groups);
            if (e < n) sq += sq1(g[e]);
        }
    }
    store_partial(sq, partials);
}

// Grid-stride form with rows (ZERO_SQNORM_ROWS = R > 0; 0, the default, keeps
// sqnorm_pass for large inputs): a fixed grid of at most ZERO_SQNORM_MAX_BLOCKS
// workgroups; per pass a workgroup reads R * kThreads consecutive groups, each
// lane R of them kThreads apart, all R loads issued together (lanes past the
// end reload the last group and drop it). One partial per workgroup, so one
// final-sum kernel. Measured on MI355X, Llama-3-70B rank 7's 8.8 G-element
// gradient in the benchmark step, two runs: sqnorm_pass 2,601-2,656 us;
// R = 4, 8, 16 over 4,096 workgroups 2,640-2,654, 2,659-2,707 and
// 2,641-2,749 us; R = 8 over 2,048 workgroups 2,616-2,666 us. Off.
#ifndef ZERO_SQNORM_ROWS
#define ZERO_SQNORM_ROWS 0
#endif
constexpr int kSqRows = ZERO_SQNORM_ROWS;

template <int R>
__global__ __launch_bounds__(kThreads) void sqnorm_rows(const uint16_t* __restrict__ g, int64_t n,
                                                        double* __restrict__ partials) {
    const int64_t groups = n / 8;
    const int64_t span = int64_t(R) * kThreads;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * span;
    const u32x4* g4 = reinterpret_cast<const u32x4*>(g);
    double sq = 0.0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * span; base < groups; base += stride) {
        u32x4 x[R];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int64_t i = base + int64_t(q) * kThreads + threadIdx.x;
            x[q] = zero::dev::ld_stream(g4 + (i < groups ? i : groups - 1));
        }
#pragma unroll
        for (int q = 0; q < R; ++q)
            if (base + int64_t(q) * kThreads + threadIdx.x < groups) sq += sq8(x[q]);
    }
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (tid < n - groups * 8) sq += sq1(g[groups * 8 + tid]);
    store_partial(sq, partials);
}

__global__ __launch_bounds__(kThreads) void sqnorm_scalar(const uint16_t* __restrict__ g, int64_t n,
                                                          double* __restrict__ partials) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    double sq = 0.0;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; e < n; e += stride)
        sq += sq1(g[e]);
    store_partial(sq, partials);
}

// Adds partials[0..count) in a fixed order into out[0]: thread t sums
// t, t+256, ... sequentially, then the fixed block tree.
__global__ __launch_bounds__(kThreads) void finish_sum(const double* __restrict__ partials,
                                                       int count, double* __restrict__ out) {
    __shared__ double lds[kThreads / zero::dev::kWave];
    // Thread t adds partials t, t + kThreads, t + 2*kThreads, ... in that
    // order; the loads of each batch of 8 are issued together.
    constexpr int kBatch = 8;
    double s = 0.0;
    for (int i0 = threadIdx.x; i0 < count; i0 += kBatch * kThreads) {
        double x[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * kThreads;
            x[k] = i < count ? partials[i] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (i0 + k * kThreads < count) s += x[k];
    }
    const double total = zero::dev::block_sum<kThreads>(s, lds);
    if (threadIdx.x == 0) out[0] = total;
}

// First level of the final sum when there are many partials (the one-pass
// reduce and squared norm): workgroup j adds partials [j * kFinishChunk, (j + 1) * kFinishChunk)
// in finish_sum's order and writes out[j]; finish_sum then adds those.
constexpr int64_t kFinishChunk = 8 * kThreads;
__global__ __launch_bounds__(kThreads) void finish_chunks(const double* __restrict__ partials,
                                                          int64_t count, double* __restrict__ out) {
    __shared__ double lds[kThreads / zero::dev::kWave];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kFinishChunk;
    const int64_t m = count - base < kFinishChunk ? count - base : kFinishChunk;
    double x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t i = threadIdx.x + int64_t(k) * kThreads;
        x[k] = i < m ? partials[base + i] : 0.0;
    }
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (threadIdx.x + int64_t(k) * kThreads < m) s += x[k];
    const double total = zero::dev::block_sum<kThreads>(s, lds);
    if (threadIdx.x == 0) out[blockIdx.x] = total;
}

__global__ void write_zero(double* out) {
    if (threadIdx.x == 0) out[0] = 0.0;
}

// Global norm from per-rank partials, in index order; the coefficient of the
// clip-by-total-norm convention, NaN when the norm is not finite.
__global__ void clip_kernel(const double* __restrict__ partials, int n, double max_norm,
                            float* __restrict__ scale) {
    // One wave: each lane loads one partial of a batch of 64 (all loads in
    // flight together), then the batch is added in index order, value by value
    // through cross-lane reads, so the sum is the sequential one.
    const int lane = threadIdx.x;
    double total = 0.0;
    for (int b = 0; b < n; b += zero::dev::kWave) {
        const double mine = b + lane < n ? partials[b + lane] : 0.0;
        const int m = n - b < zero::dev::kWave ? n - b : zero::dev::kWave;
        for (int j = 0; j < m; ++j) total += __shfl(mine, j, zero::dev::kWave);
    }
    if (lane != 0) return;
    float out;
    if (!isfinite(total)) {
        out = __builtin_nanf("");
    } else if (!(max_norm > 0.0)) {
        out = 1.0f;
    } else {
        const double coef = max_norm / (sqrt(total) + 1e-6);
        out = static_cast<float>(coef < 1.0 ? coef : 1.0);
    }
    scale[0] = out;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Past the cap, 0 keeps the grid at the cap (the last pass of the grid-stride
// loop then runs on a fraction of the lanes); 1 takes as many passes as the cap
// needs and divides the work evenly over them (every lane the same number of
// passes, within one).
#ifndef ZERO_REDUCE_BALANCED
#define ZERO_REDUCE_BALANCED 0
#endif

int grid_for(int64_t work_items, int cap) {
    int64_t blocks = (work_items + kThreads - 1) / kThreads;
    if (blocks > cap) {
        if (ZERO_REDUCE_BALANCED) {
            const int64_t passes = (blocks + cap - 1) / cap;
            blocks = (blocks + passes - 1) / passes;
        } else {
            blocks = cap;
        }
    }
    if (blocks < 1) blocks = 1;
    return static_cast<int>(blocks);
}

// Workgroups of the one-pass reduce over n elements, W words (2W elements) per lane.
int64_t pass_blocks(int64_t n, int w) {
    const int64_t units = (n + 2 * w - 1) / (2 * w);
    return (units + kThreads * kPassQ - 1) / (kThreads * kPassQ);
}

// Its partials, then the first-level sums of finish_chunks (doubles); W = 1
// has the most.
int64_t pass_partials(int64_t n) {
    const int64_t b = pass_blocks(n, 1);
    return b + (b + kFinishChunk - 1) / kFinishChunk;
}

// Words per lane of the one-pass kernel for windows of more than one load
// batch of replicas; 0 keeps those on the grid-stride kernels.
#ifndef ZERO_REDUCE_PASS_WIDE_WORDS
#define ZERO_REDUCE_PASS_WIDE_WORDS 0
#endif
// Words per lane of the one-pass kernel for at most one load batch of replicas.
#ifndef ZERO_REDUCE_PASS_WORDS
#define ZERO_REDUCE_PASS_WORDS 1
#endif

}  // namespace

extern "C" size_t zero_sqnorm_workspace_bytes(void) { return kMaxPartials * sizeof(double); }

extern "C" size_t zero_reduce_workspace_bytes(int64_t count) {
    const size_t fixed = zero_sqnorm_workspace_bytes();
    if (count < kOnePassFrom) return fixed;
    const size_t need = static_cast<size_t>(pass_partials(count)) * sizeof(double);
    return need > fixed ? need : fixed;
}

namespace {

// The reduce after its arguments (and, for the norm, the partials buffer: 8-byte
// aligned, at least zero_sqnorm_workspace_bytes()) have been checked.
zero_status reduce_shard(const zero_plan* plan, int32_t rank, const uint16_t* const* replicas,
                         int32_t n_replicas, int64_t begin, int64_t count, uint16_t* shard_grad,
                         double* sqnorm_out, double* partials, size_t workspace_bytes,
                         hipStream_t stream) {
    using zero::fail;
    ReplicaTable table{};
    for (int32_t k = 0; k < n_replicas; ++k) {
        if (replicas[k] == nullptr) return fail(ZERO_EINVAL, "zero_grad_reduce_shard: NULL replica");
        table.p[k] = replicas[k];
    }
    const int64_t shard_lo = static_cast<int64_t>(rank) * plan->shard;
    const int64_t lo = begin > shard_lo ? begin : shard_lo;
    const int64_t end = begin + count, shard_hi = shard_lo + plan->shard;
    const int64_t hi = end < shard_hi ? end : shard_hi;
    if (lo >= hi) {
        if (sqnorm_out != nullptr) {
            hipLaunchKernelGGL(write_zero, dim3(1), dim3(64), 0, stream, sqnorm_out);
            return zero::check_hip(hipGetLastError(), "zero_grad_reduce_shard launch");
        }
        return ZERO_OK;
    }
    const int64_t n = hi - lo, src_off = lo - begin;
    uint16_t* out = shard_grad + (lo - shard_lo);
    const bool norm = sqnorm_out != nullptr;
    {
        // On the stack: the no-allocation entry point comes through here too.
        const size_t bytes = static_cast<size_t>(n) * 2;
        const zero::Span wr[] = {{out, bytes, "shard_grad"},
                                 {partials, norm ? workspace_bytes : 0, "workspace"}};
        zero::Span rd[ZERO_MAX_REPLICAS];
        for (int32_t k = 0; k < n_replicas; ++k) rd[k] = {replicas[k] + src_off, bytes, "replica", k};
        const std::string clash = zero::first_overlap(wr, 2, rd, n_replicas);
        if (!clash.empty()) return fail(ZERO_EINVAL, "zero_grad_reduce_shard: " + clash);
    }
    // Large windows of at most one load batch of replicas: the one-pass
    // kernel, when every replica slice and the output are 4-byte aligned and
    // the workspace holds its partials. (With more replicas a lane makes one
    // round trip per batch of 4-byte loads, and the grid-stride kernel's
    // 16-byte loads measured faster: 64 replicas over 25 M elements, 2.66 ms
    // against 2.72 ms per 125 M-element shard.)
    const int pw = n_replicas <= kReplicaBatch ? ZERO_REDUCE_PASS_WORDS : ZERO_REDUCE_PASS_WIDE_WORDS;
    bool pass = pw > 0 && n >= kOnePassFrom && aligned(out, 4 * pw) &&
                (!norm || workspace_bytes >= static_cast<size_t>(pass_partials(n)) * sizeof(double));
    for (int32_t k = 0; k < n_replicas && pass; ++k) pass = aligned(replicas[k] + src_off, 4 * pw);
    if (pass) {
        constexpr int64_t kMaxBlocks = (int64_t(1) << 32) / kThreads - 1;
        const int64_t blocks = pass_blocks(n, pw);
        for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks) {
            const int64_t nb = blocks - b0 < kMaxBlocks ? blocks - b0 : kMaxBlocks;
            const dim3 grid(static_cast<unsigned>(nb));
            double* const part = norm ? partials + b0 : partials;
            if (norm && pw == 1)
                hipLaunchKernelGGL((reduce_pass<true, 1>), grid, dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, b0, part);
            else if (norm && pw == 2)
                hipLaunchKernelGGL((reduce_pass<true, 2>), grid, dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, b0, part);
            else if (norm)
                hipLaunchKernelGGL((reduce_pass<true, 4>), grid, dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, b0, part);
            else if (pw == 1)
                hipLaunchKernelGGL((reduce_pass<false, 1>), grid, dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, b0, part);
            else if (pw == 2)
                hipLaunchKernelGGL((reduce_pass<false, 2>), grid, dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, b0, part);
            else
                hipLaunchKernelGGL((reduce_pass<false, 4>), grid, dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, b0, part);
            zero_status st = zero::check_hip(hipGetLastError(), "zero_grad_reduce_shard launch");
            if (st != ZERO_OK) return st;
        }
        if (!norm) return ZERO_OK;
        // partials[0, blocks) -> first-level sums at partials + blocks -> the total
        const int64_t level1 = (blocks + kFinishChunk - 1) / kFinishChunk;
        hipLaunchKernelGGL(finish_chunks, dim3(static_cast<unsigned>(level1)), dim3(kThreads), 0, stream,
                           partials, blocks, partials + blocks);
        zero_status st = zero::check_hip(hipGetLastError(), "zero_grad_reduce_shard finish launch");
        if (st != ZERO_OK) return st;
        hipLaunchKernelGGL(finish_sum, dim3(1), dim3(kThreads), 0, stream, partials + blocks,
                           static_cast<int>(level1), sqnorm_out);
        return zero::check_hip(hipGetLastError(), "zero_grad_reduce_shard finish launch");
    }
    bool vec = aligned(out, 2 * kEpt);
    for (int32_t k = 0; k < n_replicas && vec; ++k) vec = aligned(replicas[k] + src_off, 2 * kEpt);
    const int blocks = grid_for(vec ? (kRows > 1 ? (n / kEpt + kRows - 1) / kRows : n / kEpt) : n,
                                ZERO_REDUCE_MAX_BLOCKS);
    if (vec) {
        const bool two = n_replicas <= kReplicaBatch && n >= kTwoGroupsFrom;
        if constexpr (kRows > 1) {
            if (norm)
                hipLaunchKernelGGL(reduce_rows<true>, dim3(blocks), dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, partials);
            else
                hipLaunchKernelGGL(reduce_rows<false>, dim3(blocks), dim3(kThreads), 0, stream, table,
                                   n_replicas, src_off, out, n, partials);
        } else if (norm && two)
            hipLaunchKernelGGL((reduce_vec<true, 2>), dim3(blocks), dim3(kThreads), 0, stream, table,
                               n_replicas, src_off, out, n, partials);
        else if (norm)
            hipLaunchKernelGGL((reduce_vec<true, 1>), dim3(blocks), dim3(kThreads), 0, stream, table,
                               n_replicas, src_off, out, n, partials);
        else if (two)
            hipLaunchKernelGGL((reduce_vec<false, 2>), dim3(blocks), dim3(kThreads), 0, stream, table,
                               n_replicas, src_off, out, n, partials);
        else
            hipLaunchKernelGGL((reduce_vec<false, 1>), dim3(blocks), dim3(kThreads), 0, stream, table,
                               n_replicas, src_off, out, n, partials);
    } else {
        if (norm)
            hipLaunchKernelGGL(reduce_scalar<true>, dim3(blocks), dim3(kThreads), 0, stream, table,
                               n_replicas, src_off, out, n, partials);
        else
            hipLaunchKernelGGL(reduce_scalar<false>, dim3(blocks), dim3(kThreads), 0, stream, table,
                               n_replicas, src_off, out, n, partials);
    }
    zero_status st = zero::check_hip(hipGetLastError(), "zero_grad_reduce_shard launch");
    if (st != ZERO_OK || !norm) return st;
    hipLaunchKernelGGL(finish_sum, dim3(1), dim3(kThreads), 0, stream, partials, blocks, sqnorm_out);
    return zero::check_hip(hipGetLastError(), "zero_grad_reduce_shard finish launch");
}


// Checks the arguments every form of the reduce shares.
zero_status check_reduce_args(const zero_plan* plan, int32_t rank, const uint16_t* const* replicas,
                              int32_t n_replicas, int64_t begin, int64_t count,
                              const uint16_t* shard_grad) {
    using zero::fail;
    if (plan == nullptr || replicas == nullptr || shard_grad == nullptr)
        return fail(ZERO_EINVAL, "zero_grad_reduce_shard: NULL plan, replicas or shard_grad");
    if (rank < 0 || rank >= plan->n_ranks)
        return fail(ZERO_EINVAL, "zero_grad_reduce_shard: rank out of range");
    if (n_replicas < 1 || n_replicas > ZERO_MAX_REPLICAS)
        return fail(ZERO_EINVAL, "zero_grad_reduce_shard: n_replicas must be 1.." +
                                     std::to_string(ZERO_MAX_REPLICAS));
    if (begin < 0 || count < 0 || begin > plan->padded || count > plan->padded - begin)
        return fail(ZERO_EINVAL, "zero_grad_reduce_shard: window outside [0, P)");
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_grad_reduce_shard(const zero_plan* plan, int32_t rank,
                                              const uint16_t* const* replicas, int32_t n_replicas,
                                              int64_t begin, int64_t count, uint16_t* shard_grad,
                                              double* sqnorm_out, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    zero_status st = check_reduce_args(plan, rank, replicas, n_replicas, begin, count, shard_grad);
    if (st != ZERO_OK) return st;
    if (sqnorm_out != nullptr) {
        if (workspace == nullptr) return fail(ZERO_EINVAL, "zero_grad_reduce_shard: NULL workspace");
        if (!aligned(workspace, 8))
            return fail(ZERO_EINVAL, "zero_grad_reduce_shard: workspace not 8-byte aligned");
        if (workspace_bytes < zero_sqnorm_workspace_bytes())
            return fail(ZERO_ENOSPACE, "zero_grad_reduce_shard: workspace too small");
    }
    return reduce_shard(plan, rank, replicas, n_replicas, begin, count, shard_grad, sqnorm_out,
                        static_cast<double*>(workspace), workspace_bytes, stream);
}

// ------------------------------------------------------------ per-tensor replicas
//
// "FSDP-1: FlatParameter and Module-Level Wrapping" places every tensor in the
// flat padded buffer; "Execution Flow for ZeRO-1", step 2, averages the rank's
// slice of it over the replicas. When the replicas are still per-tensor (as a
// backward pass leaves them), the rank's slice can be reduced from them
// directly, with no flatten of each replica first: for every segment of the
// rank's shard, elements [tensor_offset, tensor_offset + length) of tensor t in
// each replica, reduced into shard elements [shard_offset, shard_offset +
// length); the shard's padding is written as zeros. The arithmetic is
// reduce_vec's (fp32 sum in replica order, one division by R, one rounding), so
// the bits are those of zero_grad_reduce_shard over the flattened replicas.
// Per shard element: R bf16 reads and one bf16 write, (2R + 2) bytes, against
// 4R more for flattening R replicas first.
//
// The table is built once for fixed buffers: one 64-byte descriptor per piece
// (a segment, or a gap of padding), an XCD-major per-workgroup index, the
// replica pointers tensor-major (pointer of replica k's tensor t at t * R + k,
// so a workgroup's R pointers are contiguous), and a partial per workgroup for
// the squared norm. A workgroup reduces kRChunk elements of one piece, 8 per
// lane through 16-byte accesses where every replica's tensor, the offsets and
// the shard are 8-element aligned, element by element otherwise.
using zero::copy::RPieceDesc;

namespace {

// 2,048-element groups per workgroup (the descriptor lookup is paid once per
// workgroup). Measured on MI355X, GPT-2 rank 7 from 8 per-tensor replicas, two
// runs, flat plan: 1 group 49.4-49.9 us, 2 groups 50.7-50.8 us, 4 groups
// 54.7-54.8 us (Shard(0): 51.8-52.0, 52.7-52.9, 57.7-58.0 us). One stays.
#ifndef ZERO_RTABLE_GROUPS
#define ZERO_RTABLE_GROUPS 1
#endif
constexpr int kRGroups = ZERO_RTABLE_GROUPS;
constexpr int64_t kRChunk = int64_t(kThreads) * 8 * kRGroups;   // elements per workgroup
// 1: the one-pass form leaves one norm partial per wave (no LDS, no barrier;
// four times the partials); 0 (default): one per workgroup. Measured on MI355X,
// GPT-2 rank 7 from 8 per-tensor replicas, two runs: 50.4-50.5 us against
// 49.8-50.0 us (Shard(0): 51.7 against 50.9-51.1 us).
#ifndef ZERO_RTABLE_WAVE_PARTIALS
#define ZERO_RTABLE_WAVE_PARTIALS 0
#endif
constexpr int64_t kRPartialsPerBlock = ZERO_RTABLE_WAVE_PARTIALS ? kThreads / 64 : 1;
// Workgroups of the grid-stride form (0, default: one workgroup per chunk, one
// pass). Measured on MI355X, GPT-2 rank 7 from 8 per-tensor replicas, two
// runs: one pass 50.5-50.9 us; grids of 1,024, 2,048 and 4,096 workgroups
// 55.7-56.1, 55.8-56.1 and 51.9-52.1 us.
#ifndef ZERO_RTABLE_GRID
#define ZERO_RTABLE_GRID 0
#endif
// 1: the 16-byte path issues each batch of replica loads together
// (zero::dev::for_replicas); 0 (default): a guarded load per replica. Measured
// on MI355X, GPT-2 rank 7 from 8 per-tensor replicas, two runs: 51.3-51.5 us
// against 50.6-51.1 us on the flat plan, 53.5 against 51.3-51.9 us on Shard(0).
#ifndef ZERO_RTABLE_BATCHED_ISSUE
#define ZERO_RTABLE_BATCHED_ISSUE 0
#endif

// Workgroup chunk `blk` of piece d: its gradient elements, and their squares
// added to this thread's sq.
__device__ __forceinline__ void reduce_table_chunk(const RPieceDesc& d, int64_t blk,
                                                   const uint16_t* const* __restrict__ ptrs, int n_rep,
                                                   uint16_t* __restrict__ out, double& sq) {
    const int64_t start = (blk - d.first_block) * kRChunk;
    const int64_t len = d.len - start < kRChunk ? d.len - start : kRChunk;
    uint16_t* const o = out + d.dst_off + start;
    if (d.tensor < 0) {
        for (int64_t e = threadIdx.x; e < len; e += kThreads) o[e] = 0;
    } else {
        const uint16_t* const* const p = ptrs + static_cast<int64_t>(d.tensor) * n_rep;
        const int64_t src = d.src_off + start;
        const float r = static_cast<float>(n_rep);
        auto one = [&](int64_t e) {                       // element e of the chunk
            float acc = 0.0f;
            for (int k = 0; k < n_rep; ++k) acc = acc + zero::dev::bf16_to_f32(p[k][src + e]);
            const uint16_t h = static_cast<uint16_t>(zero::dev::f32_to_bf16(acc / r));
            o[e] = h;
            sq += sq1(h);
        };
        for (int g = 0; g < kRGroups; ++g) {
        const int64_t e = (static_cast<int64_t>(g) * kThreads + threadIdx.x) * 8;
        if (d.vec && e + 8 <= len) {
            float acc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#if ZERO_RTABLE_BATCHED_ISSUE
            zero::dev::for_replicas<kReplicaBatch, u32x4>(p, n_rep, src, e / 8, [&](const u32x4& x) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[2 * j] = acc[2 * j] + zero::dev::lo_bf16(x[j]);
                    acc[2 * j + 1] = acc[2 * j + 1] + zero::dev::hi_bf16(x[j]);
                }
            });
#else
            for (int k0 = 0; k0 < n_rep; k0 += kReplicaBatch) {
                u32x4 x[kReplicaBatch];
                const int kn = n_rep - k0 < kReplicaBatch ? n_rep - k0 : kReplicaBatch;
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k)
                    if (k < kn) x[k] = zero::dev::ld_stream(reinterpret_cast<const u32x4*>(p[k0 + k] + src + e));
#pragma unroll
                for (int k = 0; k < kReplicaBatch; ++k) {
                    if (k < kn) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[2 * j] = acc[2 * j] + zero::dev::lo_bf16(x[k][j]);
                            acc[2 * j + 1] = acc[2 * j + 1] + zero::dev::hi_bf16(x[k][j]);
                        }
                    }
                }
            }
#endif
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = zero::dev::pack_bf16(acc[2 * j] / r, acc[2 * j + 1] / r);
            sq += sq8(w);
            zero::dev::st_stream(reinterpret_cast<u32x4*>(o + e), w);
        } else if (d.vec) {                               // the chunk's ragged end
            for (int64_t i = e; i < len; ++i) one(i);
        } else if (g == 0) {
            for (int64_t i = threadIdx.x; i < len; i += kThreads) one(i);
        }
        }
    }
}

__global__ __launch_bounds__(kThreads) void reduce_table_kernel(const RPieceDesc* __restrict__ table,
                                                                const uint32_t* __restrict__ index,
                                                                const uint16_t* const* __restrict__ ptrs,
                                                                int n_rep, uint16_t* __restrict__ out,
                                                                int64_t blk0, int64_t per,
                                                                double* __restrict__ partials) {
    const int64_t blk = blk0 + static_cast<int64_t>(blockIdx.x);
    double sq = 0.0;
    reduce_table_chunk(table[index[zero::dev::xcd_major_entry(blk0, per)]], blk, ptrs, n_rep, out, sq);
    if (partials == nullptr) return;
#if ZERO_RTABLE_WAVE_PARTIALS
    // one partial per wave, in (workgroup, wave) order: no LDS, no barrier
    const double w = zero::dev::wave_sum(sq);
    if (threadIdx.x % zero::dev::kWave == 0)
        partials[blk * (kThreads / zero::dev::kWave) + threadIdx.x / zero::dev::kWave] = w;
#else
    store_partial(sq, partials + blk0);
#endif
}

// Grid-stride form (one launch of at most kTableLaunchBlocks chunks): workgroup
// x takes chunks x, x + G, x + 2G, ... (G = gridDim.x), each found through the
// launch's XCD-major index, and leaves one partial.
__global__ __launch_bounds__(kThreads) void reduce_table_stride_kernel(
        const RPieceDesc* __restrict__ table, const uint32_t* __restrict__ index,
        const uint16_t* const* __restrict__ ptrs, int n_rep, uint16_t* __restrict__ out,
        int64_t blocks, int64_t per, double* __restrict__ partials) {
    double sq = 0.0;
    for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x)
        reduce_table_chunk(table[index[(blk & 7) * per + (blk >> 3)]], blk, ptrs, n_rep, out, sq);
    if (partials != nullptr) store_partial(sq, partials);
}

}  // namespace

struct zero_reduce_table {
    int device = -1;
    void* mem = nullptr;            // descriptors, index, replica pointers, partials
    const RPieceDesc* table = nullptr;
    const uint32_t* index = nullptr;
    const uint16_t* const* ptrs = nullptr;
    double* partials = nullptr;     // blocks, then the first-level sums
    uint16_t* out = nullptr;
    int32_t n_rep = 0;
    int64_t blocks = 0;
};

extern "C" zero_status zero_reduce_table_create(const zero_plan* plan, int32_t rank,
                                                const uint16_t* const* replica_tensors,
                                                int32_t n_replicas, uint16_t* shard_grad,
                                                zero_reduce_table** out) {
    using zero::fail;
    static const char* const who = "zero_reduce_table_create";
    zero::clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "zero_reduce_table_create: NULL out");
    *out = nullptr;
    if (plan == nullptr || replica_tensors == nullptr)
        return fail(ZERO_EINVAL, "zero_reduce_table_create: NULL plan or replica_tensors");
    if (rank < 0 || rank >= plan->n_ranks)
        return fail(ZERO_EINVAL, "zero_reduce_table_create: rank out of range");
    if (n_replicas < 1 || n_replicas > ZERO_MAX_REPLICAS)
        return fail(ZERO_EINVAL, "zero_reduce_table_create: n_replicas must be 1.." +
                                     std::to_string(ZERO_MAX_REPLICAS));
    if (plan->shard > 0 && shard_grad == nullptr)
        return fail(ZERO_EINVAL, "zero_reduce_table_create: NULL shard_grad");
    std::vector<RPieceDesc> descs;
    std::vector<uint32_t> index;
    std::vector<const uint16_t*> ptrs;
    int64_t blocks = 0;
    try {
        const zero_status cs = zero::copy::reduce_table_contents(
            plan, rank, replica_tensors, n_replicas, shard_grad, kRChunk, &descs, &index, &ptrs,
            &blocks, who);
        if (cs != ZERO_OK) return cs;
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, std::string(who) + ": host allocation failed");
    }
    zero_reduce_table* tab = nullptr;
    try {
        tab = new zero_reduce_table;
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, std::string(who) + ": host allocation failed");
    }
    tab->out = shard_grad;
    tab->n_rep = n_replicas;
    tab->blocks = blocks;
    zero_status st = ZERO_OK;
    if (blocks > 0) {                // an empty shard needs no device
        auto up = [](size_t b) { return (b + 255) / 256 * 256; };
        const size_t desc_bytes = up(descs.size() * sizeof(RPieceDesc));
        const size_t index_bytes = up(index.size() * sizeof(uint32_t));
        const size_t ptr_bytes = up(ptrs.size() * sizeof(const uint16_t*));
        const int64_t n_part = blocks * kRPartialsPerBlock;
        const int64_t level1 = (n_part + kFinishChunk - 1) / kFinishChunk;
        const size_t part_bytes = static_cast<size_t>(n_part + level1) * sizeof(double);
        st = zero::check_hip(hipGetDevice(&tab->device), who);
        if (st == ZERO_OK)
            st = zero::check_hip(hipMalloc(&tab->mem, desc_bytes + index_bytes + ptr_bytes + part_bytes), who);
        if (st == ZERO_OK) {
            char* m = static_cast<char*>(tab->mem);
            tab->table = reinterpret_cast<const RPieceDesc*>(m);
            tab->index = reinterpret_cast<const uint32_t*>(m + desc_bytes);
            tab->ptrs = reinterpret_cast<const uint16_t* const*>(m + desc_bytes + index_bytes);
            tab->partials = reinterpret_cast<double*>(m + desc_bytes + index_bytes + ptr_bytes);
            st = zero::check_hip(hipMemcpy(m, descs.data(), descs.size() * sizeof(RPieceDesc),
                                           hipMemcpyHostToDevice), who);
            if (st == ZERO_OK)
                st = zero::check_hip(hipMemcpy(m + desc_bytes, index.data(), index.size() * sizeof(uint32_t),
                                               hipMemcpyHostToDevice), who);
            if (st == ZERO_OK)
                st = zero::check_hip(hipMemcpy(m + desc_bytes + index_bytes, ptrs.data(),
                                               ptrs.size() * sizeof(const uint16_t*), hipMemcpyHostToDevice),
                                     who);
        }
    }
    if (st != ZERO_OK) {
        if (tab->mem) (void)hipFree(tab->mem);
        delete tab;
        return st;
    }
    *out = tab;
    return ZERO_OK;
}

extern "C" zero_status zero_reduce_table_run(const zero_reduce_table* table, double* sqnorm_out,
                                             hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (table == nullptr) return fail(ZERO_EINVAL, "zero_reduce_table_run: NULL table");
    if (table->blocks == 0) {
        if (sqnorm_out == nullptr) return ZERO_OK;
        hipLaunchKernelGGL(write_zero, dim3(1), dim3(64), 0, stream, sqnorm_out);
        return zero::check_hip(hipGetLastError(), "zero_reduce_table_run launch");
    }
    int dev = -1;
    zero_status st = zero::check_hip(hipGetDevice(&dev), "zero_reduce_table_run: hipGetDevice");
    if (st != ZERO_OK) return st;
    if (dev != table->device)
        return fail(ZERO_EINVAL, "zero_reduce_table_run: the table lives on device " +
                                     std::to_string(table->device) + ", the current device is " +
                                     std::to_string(dev));
    double* const parts = sqnorm_out != nullptr ? table->partials : nullptr;
    // A dispatch holds fewer than 2^32 work-items: longer tables take several launches.
    constexpr int64_t kMaxBlocks = zero::kTableLaunchBlocks;
    int64_t n_parts = table->blocks * kRPartialsPerBlock;
    if (ZERO_RTABLE_GRID > 0 && !ZERO_RTABLE_WAVE_PARTIALS && table->blocks <= kMaxBlocks) {
        n_parts = table->blocks < ZERO_RTABLE_GRID ? table->blocks : ZERO_RTABLE_GRID;
        hipLaunchKernelGGL(reduce_table_stride_kernel, dim3(static_cast<unsigned>(n_parts)), dim3(kThreads),
                           0, stream, table->table, table->index, table->ptrs, table->n_rep, table->out,
                           table->blocks, (table->blocks + 7) / 8, parts);
        st = zero::check_hip(hipGetLastError(), "zero_reduce_table_run launch");
        if (st != ZERO_OK) return st;
    } else for (int64_t b0 = 0; b0 < table->blocks; b0 += kMaxBlocks) {
        const int64_t nb = table->blocks - b0 < kMaxBlocks ? table->blocks - b0 : kMaxBlocks;
        const int64_t per = (nb + 7) / 8;
        hipLaunchKernelGGL(reduce_table_kernel, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, stream,
                           table->table, table->index, table->ptrs, table->n_rep, table->out, b0, per,
                           parts);
        st = zero::check_hip(hipGetLastError(), "zero_reduce_table_run launch");
        if (st != ZERO_OK) return st;
    }
    if (sqnorm_out == nullptr) return ZERO_OK;
    // partials[0, n_parts) -> first-level sums after them -> the total
    const int64_t level1 = (n_parts + kFinishChunk - 1) / kFinishChunk;
    hipLaunchKernelGGL(finish_chunks, dim3(static_cast<unsigned>(level1)), dim3(kThreads), 0, stream,
                       table->partials, n_parts, table->partials + n_parts);
    st = zero::check_hip(hipGetLastError(), "zero_reduce_table_run finish launch");
    if (st != ZERO_OK) return st;
    hipLaunchKernelGGL(finish_sum, dim3(1), dim3(kThreads), 0, stream, table->partials + n_parts,
                       static_cast<int>(level1), sqnorm_out);
    return zero::check_hip(hipGetLastError(), "zero_reduce_table_run finish launch");
}

extern "C" int64_t zero_reduce_table_blocks(const zero_reduce_table* table) {
    return table ? table->blocks : -1;
}

extern "C" void zero_reduce_table_free(zero_reduce_table* table) {
    if (!table) return;
    if (table->mem) (void)hipFree(table->mem);
    delete table;
}

// ------------------------------------------------------------ no allocation
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the reduce with its norm partials in a library-owned device array.
// Each device holds its own copy of `scratch` from the library's load until the
// process ends; host code never passes the array's name to a kernel (on the
// host it is only a stand-in), but the address hipGetSymbolAddress gives for
// the current device, looked up once per device and kept.
constexpr size_t kStaticScratchBytes = ZERO_NOALLOC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes >= kMaxPartials * sizeof(double),
              "the scratch holds the grid-stride kernels' partials");
static __device__ __align__(256) double scratch[kStaticScratchBytes / sizeof(double)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`.
zero_status device_scratch(double** out) {
    int dev = -1;
    zero_status st = zero::check_hip(hipGetDevice(&dev), "zero_grad_reduce_shard_noalloc: hipGetDevice");
    if (st != ZERO_OK) return st;
    if (dev < 0 || dev >= kMaxDevices)
        return zero::fail(ZERO_ERANGE, "zero_grad_reduce_shard_noalloc: device index " +
                                           std::to_string(dev) + " past " + std::to_string(kMaxDevices - 1));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        st = zero::check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                             "zero_grad_reduce_shard_noalloc: hipGetSymbolAddress");
        if (st != ZERO_OK) return st;
        if (p == nullptr)
            return zero::fail(ZERO_EHIP, "zero_grad_reduce_shard_noalloc: no device address for the scratch");
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<double*>(g_scratch_ptr[dev]);
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_grad_reduce_shard_noalloc(const zero_plan* plan, int32_t rank,
                                                      const uint16_t* const* replicas,
                                                      int32_t n_replicas, int64_t begin,
                                                      int64_t count, uint16_t* shard_grad,
                                                      double* sqnorm_out, hipStream_t stream) {
    zero::clear_error();
    zero_status st = check_reduce_args(plan, rank, replicas, n_replicas, begin, count, shard_grad);
    if (st != ZERO_OK) return st;
    double* partials = nullptr;
    if (sqnorm_out != nullptr) {
        st = device_scratch(&partials);
        if (st != ZERO_OK) return st;
    }
    // The partials need no clearing: each kernel writes every slot it later reads.
    return reduce_shard(plan, rank, replicas, n_replicas, begin, count, shard_grad, sqnorm_out,
                        partials, sqnorm_out != nullptr ? kStaticScratchBytes : 0, stream);
}

extern "C" zero_status zero_grad_sqnorm(const uint16_t* grad, int64_t n, double* sqnorm_out,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "zero_grad_sqnorm: n < 0");
    if (sqnorm_out == nullptr || (n > 0 && grad == nullptr) || workspace == nullptr)
        return fail(ZERO_EINVAL, "zero_grad_sqnorm: NULL pointer");
    if (!aligned(workspace, 8))
        return fail(ZERO_EINVAL, "zero_grad_sqnorm: workspace not 8-byte aligned");
    if (workspace_bytes < zero_sqnorm_workspace_bytes())
        return fail(ZERO_ENOSPACE, "zero_grad_sqnorm: workspace too small");
    double* partials = static_cast<double*>(workspace);
    if (n == 0) {
        hipLaunchKernelGGL(write_zero, dim3(1), dim3(64), 0, stream, sqnorm_out);
        return zero::check_hip(hipGetLastError(), "zero_grad_sqnorm launch");
    }
    const bool vec = aligned16(grad);
    // Large aligned inputs with a workspace for a partial per workgroup: one pass.
    const int64_t lanes = n / 8 + n % 8;
    const int64_t pblocks = (lanes + kThreads * kSqPassGroups - 1) / (kThreads * kSqPassGroups);
    const int64_t plevel1 = (pblocks + kFinishChunk - 1) / kFinishChunk;
    if constexpr (kSqRows > 0) {
        if (vec && n >= kOnePassFrom) {
            const int64_t span = int64_t(kSqRows) * kThreads;
            const int64_t want = (n / 8 + span - 1) / span;
            const int blocks = static_cast<int>(want < ZERO_SQNORM_MAX_BLOCKS ? want : ZERO_SQNORM_MAX_BLOCKS);
            hipLaunchKernelGGL(sqnorm_rows<kSqRows>, dim3(blocks), dim3(kThreads), 0, stream, grad, n,
                               partials);
            zero_status st = zero::check_hip(hipGetLastError(), "zero_grad_sqnorm launch");
            if (st != ZERO_OK) return st;
            hipLaunchKernelGGL(finish_sum, dim3(1), dim3(kThreads), 0, stream, partials, blocks, sqnorm_out);
            return zero::check_hip(hipGetLastError(), "zero_grad_sqnorm finish launch");
        }
    }
    if (vec && n >= kOnePassFrom &&
        workspace_bytes >= static_cast<size_t>(pblocks + plevel1) * sizeof(double)) {
        constexpr int64_t kMaxBlocks = (int64_t(1) << 32) / kThreads - 1;
        for (int64_t b0 = 0; b0 < pblocks; b0 += kMaxBlocks) {
            const int64_t nb = pblocks - b0 < kMaxBlocks ? pblocks - b0 : kMaxBlocks;
            hipLaunchKernelGGL(sqnorm_pass, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, stream,
                               grad, n, b0, partials + b0);
            zero_status st = zero::check_hip(hipGetLastError(), "zero_grad_sqnorm launch");
            if (st != ZERO_OK) return st;
        }
        hipLaunchKernelGGL(finish_chunks, dim3(static_cast<unsigned>(plevel1)), dim3(kThreads), 0, stream,
                           partials, pblocks, partials + pblocks);
        zero_status st = zero::check_hip(hipGetLastError(), "zero_grad_sqnorm finish launch");
        if (st != ZERO_OK) return st;
        hipLaunchKernelGGL(finish_sum, dim3(1), dim3(kThreads), 0, stream, partials + pblocks,
                           static_cast<int>(plevel1), sqnorm_out);
        return zero::check_hip(hipGetLastError(), "zero_grad_sqnorm finish launch");
    }
    const int blocks = grid_for(vec ? n / 8 : n, ZERO_SQNORM_MAX_BLOCKS);
    if (vec)
        hipLaunchKernelGGL(sqnorm_vec, dim3(blocks), dim3(kThreads), 0, stream, grad, n, partials);
    else
        hipLaunchKernelGGL(sqnorm_scalar, dim3(blocks), dim3(kThreads), 0, stream, grad, n, partials);
    zero_status st = zero::check_hip(hipGetLastError(), "zero_grad_sqnorm launch");
    if (st != ZERO_OK) return st;
    hipLaunchKernelGGL(finish_sum, dim3(1), dim3(kThreads), 0, stream, partials, blocks, sqnorm_out);
    return zero::check_hip(hipGetLastError(), "zero_grad_sqnorm finish launch");
}

extern "C" zero_status zero_clip_scale(const double* partials, int32_t n_partials, double max_norm,
                                       float* scale_out, hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (partials == nullptr || scale_out == nullptr)
        return fail(ZERO_EINVAL, "zero_clip_scale: NULL pointer");
    if (n_partials < 1 || n_partials > 65536)
        return fail(ZERO_EINVAL, "zero_clip_scale: n_partials must be 1..65536");
    if (std::isnan(max_norm)) return fail(ZERO_EINVAL, "zero_clip_scale: max_norm is NaN");
    hipLaunchKernelGGL(clip_kernel, dim3(1), dim3(64), 0, stream, partials, n_partials, max_norm,
                       scale_out);
    return zero::check_hip(hipGetLastError(), "zero_clip_scale launch");
}
