// Fused mixed-precision AdamW update of one rank's shard (gfx950).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...": section "Static Memory Allocation" fixes the
// state (fp32 master, m_t, v_t; 16-bit parameters), "Execution Flow for
// ZeRO-1" steps 3-4 the work (update the own slice, emit 16-bit parameters),
// and "ZeRO-Offload Mechanics" its cost (O(1) per parameter). The update
// formula follows decoupled-weight-decay AdamW with bias correction; the
// per-element order of fp32 operations is fixed (see the ABI header) and the
// library is compiled without floating-point contraction, so results do not
// depend on the launch shape.
//
// Memory: 28 bytes per element (read 12 fp32 + 2 bf16, write 12 fp32 + 2
// bf16), about 15 flops: HBM-bound by a factor of ~40 against the fp32
// vector ridge point, so no matrix cores. Each lane updates one element
// (dword per fp32 array, short for the bf16 gradient and parameter) with
// non-temporal loads and write-through stores. The grid covers the shard with one element per lane, in
// one dispatch (rows of workgroups past 2^32 work-items): measured on MI355X,
// short-lived waves with narrow accesses sustain more bandwidth on this
// 4-read/4-write pattern than wide vectors or a persistent loop. The same
// kernel serves any pointer alignment. Indices are 64-bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <string>
#include <vector>

#include "device_common.hpp"
#include "internal.hpp"
#include "schedule.hpp"

#pragma clang fp contract(off)

namespace {

using zero::dev::f32x4;
using zero::dev::u32x2;

#ifndef ZERO_ADAMW_THREADS
#define ZERO_ADAMW_THREADS 256
#endif
// Elements per lane: 1 (default), 2 or 4. Narrow per-lane accesses sustain more
// bandwidth on this 8-stream pattern: measured on MI355X at 125M-1G elements,
// 1 element per lane runs at ~6.55 TB/s, 2 at ~6.3, 4 at ~5.7.
#ifndef ZERO_ADAMW_EPT
#define ZERO_ADAMW_EPT 1
#endif
constexpr int kThreads = ZERO_ADAMW_THREADS;
constexpr int kEpt = ZERO_ADAMW_EPT;
static_assert(kEpt == 1 || kEpt == 2 || kEpt == 4, "1, 2 or 4 elements per lane");

// The per-step scalars, computed on the host (schedule.hpp).
using AdamScalars = zero::adam::StepScalars;

// One element, in the documented order; every line is one IEEE fp32 operation.
__device__ __forceinline__ void adam_elem(float& p, float& m, float& v, float g,
                                          const AdamScalars& c) {
    const float bm = c.beta1 * m;
    const float gm = c.one_minus_beta1 * g;
    m = bm + gm;
    const float bv = c.beta2 * v;
    const float gg = g * g;
    const float gv = c.one_minus_beta2 * gg;
    v = bv + gv;
    p = p * c.decay;
    const float root = sqrtf(v);
    const float denom = root / c.sqrt_bc2 + c.eps;
    const float ratio = m / denom;
    p = p - c.step_size * ratio;
}

__device__ __forceinline__ float read_clip(const float* clip_scale) {
    return clip_scale != nullptr ? *clip_scale : 1.0f;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int E> struct Lane;   // one lane's elements and their access widths

// Addressing of the one-element lanes: 0 (default) gives each access its own
// 64-bit address; 1 addresses every array through the wave's first element (a
// wave-uniform base) plus the lane's distance from it, shared by the 8 accesses.
#ifndef ZERO_ADAMW_WAVE_BASE
#define ZERO_ADAMW_WAVE_BASE 0
#endif

template <> struct Lane<1> {
    static __device__ __forceinline__ void update(float* P, float* M, float* V, const uint16_t* G,
                                                  uint16_t* O, int64_t i, float clip,
                                                  const AdamScalars& c) {
#if ZERO_ADAMW_WAVE_BASE
        // Active lanes of a wave hold consecutive i, so i - w0 < 64.
        const int64_t w0 = zero::dev::first_lane(i);
        const uint32_t d = static_cast<uint32_t>(i - w0);
        float p = __builtin_bit_cast(float, zero::dev::ld_stream_at_b32(P + w0, d * 4));
        float m = __builtin_bit_cast(float, zero::dev::ld_stream_at_b32(M + w0, d * 4));
        float v = __builtin_bit_cast(float, zero::dev::ld_stream_at_b32(V + w0, d * 4));
        const uint16_t g = zero::dev::ld_stream_at_b16(G + w0, d * 2);
        adam_elem(p, m, v, zero::dev::bf16_to_f32(g) * clip, c);
        zero::dev::st_stream_at(P + w0, d * 4, p);
        zero::dev::st_stream_at(M + w0, d * 4, m);
        zero::dev::st_stream_at(V + w0, d * 4, v);
        zero::dev::st_stream_at(O + w0, d * 2, static_cast<uint16_t>(zero::dev::f32_to_bf16(p)));
#else
        float p = zero::dev::ld_stream(P + i);
        float m = zero::dev::ld_stream(M + i);
        float v = zero::dev::ld_stream(V + i);
        const uint16_t g = zero::dev::ld_stream(G + i);
        adam_elem(p, m, v, zero::dev::bf16_to_f32(g) * clip, c);
        zero::dev::st_stream(P + i, p);
        zero::dev::st_stream(M + i, m);
        zero::dev::st_stream(V + i, v);
        zero::dev::st_stream(O + i, static_cast<uint16_t>(zero::dev::f32_to_bf16(p)));
#endif
    }
};

template <> struct Lane<2> {
    static __device__ __forceinline__ void update(float* P, float* M, float* V, const uint16_t* G,
                                                  uint16_t* O, int64_t i, float clip,
                                                  const AdamScalars& c) {
        f32x2 p = zero::dev::ld_stream(reinterpret_cast<f32x2*>(P) + i);
        f32x2 m = zero::dev::ld_stream(reinterpret_cast<f32x2*>(M) + i);
        f32x2 v = zero::dev::ld_stream(reinterpret_cast<f32x2*>(V) + i);
        const uint32_t g = zero::dev::ld_stream(reinterpret_cast<const uint32_t*>(G) + i);
        const float gs[2] = {zero::dev::lo_bf16(g), zero::dev::hi_bf16(g)};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float pj = p[j], mj = m[j], vj = v[j];
            adam_elem(pj, mj, vj, gs[j] * clip, c);
            p[j] = pj;
            m[j] = mj;
            v[j] = vj;
        }
        zero::dev::st_stream(reinterpret_cast<f32x2*>(P) + i, p);
        zero::dev::st_stream(reinterpret_cast<f32x2*>(M) + i, m);
        zero::dev::st_stream(reinterpret_cast<f32x2*>(V) + i, v);
        zero::dev::st_stream(reinterpret_cast<uint32_t*>(O) + i, zero::dev::pack_bf16(p[0], p[1]));
    }
};

template <> struct Lane<4> {
    static __device__ __forceinline__ void update(float* P, float* M, float* V, const uint16_t* G,
                                                  uint16_t* O, int64_t i, float clip,
                                                  const AdamScalars& c) {
        f32x4 p = zero::dev::ld_stream(reinterpret_cast<f32x4*>(P) + i);
        f32x4 m = zero::dev::ld_stream(reinterpret_cast<f32x4*>(M) + i);
        f32x4 v = zero::dev::ld_stream(reinterpret_cast<f32x4*>(V) + i);
        const u32x2 g = zero::dev::ld_stream(reinterpret_cast<const u32x2*>(G) + i);
        const float gs[4] = {zero::dev::lo_bf16(g.x), zero::dev::hi_bf16(g.x),
                             zero::dev::lo_bf16(g.y), zero::dev::hi_bf16(g.y)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float pj = p[j], mj = m[j], vj = v[j];
            adam_elem(pj, mj, vj, gs[j] * clip, c);
            p[j] = pj;
            m[j] = mj;
            v[j] = vj;
        }
        zero::dev::st_stream(reinterpret_cast<f32x4*>(P) + i, p);
        zero::dev::st_stream(reinterpret_cast<f32x4*>(M) + i, m);
        zero::dev::st_stream(reinterpret_cast<f32x4*>(V) + i, v);
        const u32x2 out = {zero::dev::pack_bf16(p[0], p[1]), zero::dev::pack_bf16(p[2], p[3])};
        zero::dev::st_stream(reinterpret_cast<u32x2*>(O) + i, out);
    }
};

// Grid shape: 0 (default) covers the shard once, a lane per lane group; k > 0
// caps the grid at k workgroups per compute unit, each lane striding over the
// shard (a persistent grid sized to the chip). Measured on MI355X: one pass is
// faster on this 4-read/4-write pattern (the A/B runs are in the profiles).
#ifndef ZERO_ADAMW_PERSIST
#define ZERO_ADAMW_PERSIST 0
#endif
constexpr int kPersistPerCu = ZERO_ADAMW_PERSIST;

// Lane groups [0, n/E) of E consecutive elements, then the n % E tail one
// element per lane. For E > 1 the pointers are aligned to E elements.
template <int E>
__device__ __forceinline__ void adamw_body(float* __restrict__ master, float* __restrict__ m,
                                           float* __restrict__ v, const uint16_t* __restrict__ grad,
                                           uint16_t* __restrict__ param, int64_t n,
                                           const AdamScalars& c, float clip) {
    const int64_t groups = n / E;
    // The grid is one row of workgroups, or, past the 2^32 work-items one grid
    // dimension holds, several rows; the dispatcher issues them row after row,
    // so workgroup blockIdx.y * gridDim.x + blockIdx.x covers the shard in order.
    const int64_t blk = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t tid = blk * kThreads + threadIdx.x;
    if (kPersistPerCu > 0) {
        const int64_t stride = static_cast<int64_t>(gridDim.x) * gridDim.y * kThreads;
        for (int64_t i = tid; i < groups; i += stride) Lane<E>::update(master, m, v, grad, param, i, clip, c);
    } else {
        // The host launches a lane per group (and per tail element): one pass
        // (measured 1-2% faster than a grid-stride loop at 15.6 M-125 M elements).
        if (tid < groups) Lane<E>::update(master, m, v, grad, param, tid, clip, c);
    }
    if (E > 1) {
        const int64_t tail = n - groups * E;
        if (tid < tail) Lane<1>::update(master, m, v, grad, param, groups * E + tid, clip, c);
    }
}

template <int E>
__global__ __launch_bounds__(kThreads) void adamw_kernel(float* __restrict__ master,
                                                         float* __restrict__ m,
                                                         float* __restrict__ v,
                                                         const uint16_t* __restrict__ grad,
                                                         uint16_t* __restrict__ param, int64_t n,
                                                         AdamScalars c,
                                                         const float* __restrict__ clip_scale) {
    const float clip = read_clip(clip_scale);
    if (!isfinite(clip)) return;
    adamw_body<E>(master, m, v, grad, param, n, c, clip);
}

// A step schedule's device state: the scalars of the next step to apply and
// the number of updates applied so far. The scheduled AdamW reads `next`; the
// advance kernel, once per step, moves both on.
struct alignas(64) AdamState {
    AdamScalars next;
    int64_t applied;
    int64_t unused[3];
};
static_assert(sizeof(AdamState) == 64, "one 64-byte state");

// The flat update with the step's scalars read from the schedule's state (one
// 32-byte load per wave, beside the clip coefficient's), so a captured graph
// replays successive steps.
template <int E>
__global__ __launch_bounds__(kThreads) void adamw_sched_kernel(float* __restrict__ master,
                                                               float* __restrict__ m,
                                                               float* __restrict__ v,
                                                               const uint16_t* __restrict__ grad,
                                                               uint16_t* __restrict__ param, int64_t n,
                                                               const AdamState* __restrict__ state,
                                                               const float* __restrict__ clip_scale) {
    const float clip = read_clip(clip_scale);
    if (!isfinite(clip)) return;
    const AdamScalars c = state->next;
    adamw_body<E>(master, m, v, grad, param, n, c, clip);
}

// One lane: after a step's updates, counts the step as applied and loads the
// following step's scalars, table[min(t, length) - 1] for step t. A
// non-finite clip coefficient (the updates skipped) leaves the state as it is.
__global__ void adamw_advance_kernel(AdamState* __restrict__ state, const AdamScalars* __restrict__ table,
                                     int64_t length, const float* __restrict__ clip_scale) {
    if (threadIdx.x != 0 || !isfinite(read_clip(clip_scale))) return;
    const int64_t applied = state->applied + 1;
    const int64_t next = applied + 1;
    state->next = table[(next < length ? next : length) - 1];
    state->applied = applied;
}

// Multi-tensor form: a ragged list of tensors, each with its own five arrays,
// in one launch per kMtTensors tensors. The descriptors travel in the kernel
// arguments; workgroup b finds its tensor by a binary search over the
// per-tensor workgroup prefix and updates one element per lane with the same
// per-element code as the flat kernel (so the bits are the same).
constexpr int kMtTensors = 78;
// Elements per lane in the multi-tensor kernel: a workgroup covers kMtPer
// rows of kThreads elements (each row one coalesced access per array), so its
// tensor lookup is paid once per kMtPer * kThreads elements.
#ifndef ZERO_MT_ELEMS_PER_LANE
#define ZERO_MT_ELEMS_PER_LANE 2
#endif
constexpr int kMtPer = ZERO_MT_ELEMS_PER_LANE;
constexpr int64_t kMtChunk = int64_t(kThreads) * kMtPer;

struct MtBatch {
    float* p[kMtTensors];
    float* m[kMtTensors];
    float* v[kMtTensors];
    const uint16_t* g[kMtTensors];
    uint16_t* o[kMtTensors];
    int64_t n[kMtTensors];
    int32_t first_block[kMtTensors + 1];
    int32_t count;
};
static_assert(sizeof(MtBatch) <= 4096, "kernel arguments are limited to 4 KB");

// One workgroup's share of tensor (P, M, V, G, O) of n elements: lane element
// base + k * kThreads for k < kMtPer, the flat kernel's per-element code.
__device__ __forceinline__ void mt_update(float* __restrict__ P, float* __restrict__ M,
                                          float* __restrict__ V, const uint16_t* __restrict__ G,
                                          uint16_t* __restrict__ O, int64_t n, int64_t base,
                                          const AdamScalars& c, const float* __restrict__ clip_scale) {
    float p[kMtPer], m[kMtPer], v[kMtPer], g[kMtPer];
#pragma unroll
    for (int k = 0; k < kMtPer; ++k) {          // every load first
        const int64_t i = base + int64_t(k) * kThreads;
        if (i < n) {
            p[k] = zero::dev::ld_stream(P + i);
            m[k] = zero::dev::ld_stream(M + i);
            v[k] = zero::dev::ld_stream(V + i);
            g[k] = zero::dev::bf16_to_f32(zero::dev::ld_stream(G + i));
        }
    }
    // The coefficient is read after the loads are issued, so its latency does
    // not add to the descriptor lookup's (measured 2% faster on the 148-tensor
    // GPT-2 list). A skipped step still writes nothing.
    const float clip = read_clip(clip_scale);
    if (!isfinite(clip)) return;
#pragma unroll
    for (int k = 0; k < kMtPer; ++k) {
        const int64_t i = base + int64_t(k) * kThreads;
        if (i < n) {
            adam_elem(p[k], m[k], v[k], g[k] * clip, c);
            zero::dev::st_stream(P + i, p[k]);
            zero::dev::st_stream(M + i, m[k]);
            zero::dev::st_stream(V + i, v[k]);
            zero::dev::st_stream(O + i, static_cast<uint16_t>(zero::dev::f32_to_bf16(p[k])));
        }
    }
}

__global__ __launch_bounds__(kThreads) void adamw_multi_kernel(MtBatch b, AdamScalars c,
                                                               const float* __restrict__ clip_scale) {
    const int32_t blk = static_cast<int32_t>(blockIdx.x);
    int lo = 0, hi = b.count - 1;              // t with first_block[t] <= blk < first_block[t + 1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (b.first_block[mid] <= blk) lo = mid; else hi = mid - 1;
    }
    const int t = lo;
    mt_update(b.p[t], b.m[t], b.v[t], b.g[t], b.o[t], b.n[t],
              static_cast<int64_t>(blk - b.first_block[t]) * kMtChunk + threadIdx.x, c, clip_scale);
}

// Device-resident form of the list, for a fixed list updated every step: one
// 64-byte descriptor per non-empty tensor and, per workgroup, the index of its
// descriptor. A workgroup then finds its tensor with two dependent scalar
// loads instead of a binary search, and the whole list goes out in one launch
// (the kernel arguments hold no table).
struct alignas(64) MtDesc {
    float* p;
    float* m;
    float* v;
    const uint16_t* g;
    uint16_t* o;
    int64_t n;
    int64_t first_block;
    int64_t unused;
};
static_assert(sizeof(MtDesc) == 64, "one 64-byte descriptor per tensor");

// 1: the table holds one descriptor copy per workgroup (in the index's
// XCD-major order), so a workgroup finds its tensor with one scalar load
// instead of two dependent ones; 0 (default): one descriptor per tensor and a
// per-workgroup index. Measured on MI355X, GPT-2 rank 7's 148 Shard(0) chunks,
// three runs: 71.6-71.8 us against 71.4-71.6 us in the step; no gain.
#ifndef ZERO_MT_DESC_PER_WG
#define ZERO_MT_DESC_PER_WG 0
#endif

__global__ __launch_bounds__(kThreads) void adamw_table_kernel(const MtDesc* __restrict__ table,
                                                               const uint32_t* __restrict__ index,
                                                               int64_t blk0, int64_t per, AdamScalars c,
                                                               const float* __restrict__ clip_scale) {
    const int64_t blk = blk0 + static_cast<int64_t>(blockIdx.x);
#if ZERO_MT_DESC_PER_WG
    (void)index;
    const MtDesc d = table[zero::dev::xcd_major_entry(blk0, per)];
#else
    const MtDesc d = table[index[zero::dev::xcd_major_entry(blk0, per)]];
#endif
    mt_update(d.p, d.m, d.v, d.g, d.o, d.n, (blk - d.first_block) * kMtChunk + threadIdx.x, c,
              clip_scale);
}

// The table form with the step's scalars read from a schedule's state (used
// after the element loads are issued, as the clip coefficient is).
__global__ __launch_bounds__(kThreads) void adamw_table_sched_kernel(const MtDesc* __restrict__ table,
                                                                     const uint32_t* __restrict__ index,
                                                                     int64_t blk0, int64_t per,
                                                                     const AdamState* __restrict__ state,
                                                                     const float* __restrict__ clip_scale) {
    const int64_t blk = blk0 + static_cast<int64_t>(blockIdx.x);
#if ZERO_MT_DESC_PER_WG
    (void)index;
    const MtDesc d = table[zero::dev::xcd_major_entry(blk0, per)];
#else
    const MtDesc d = table[index[zero::dev::xcd_major_entry(blk0, per)]];
#endif
    mt_update(d.p, d.m, d.v, d.g, d.o, d.n, (blk - d.first_block) * kMtChunk + threadIdx.x, state->next,
              clip_scale);
}

// Reduce and update in one pass, for a step whose clip coefficient is known
// before the update (no clipping, or a coefficient the caller has): lane e
// averages element e of the R replicas exactly as the reduce does (an fp32 sum
// in replica order, one fp32 division by R, one rounding to bf16), optionally
// stores that bf16 gradient, and updates element e of the shard with
// adam_elem. The averaged gradient never goes through HBM: per element 2R + 24
// + 2 bytes instead of the reduce's 2R + 2 plus AdamW's 28. One element per
// lane (2-byte replica loads, 4-byte state accesses) in a one-pass grid of
// rows, as the flat AdamW; replicas are loaded 8 at a time.
struct FusedReplicas {
    const uint16_t* p[ZERO_MAX_REPLICAS];
};
// Replica loads in flight per lane in the one-pass reduce and AdamW. Measured
// on MI355X, 164 M-element shards of 8 replicas: 4 in flight 1,096 us, 8 1,054
// us, 16 1,158 us per shard; 8 is also the fastest with 64 replicas.
#ifndef ZERO_FUSED_BATCH
#define ZERO_FUSED_BATCH 8
#endif
constexpr int kFusedBatch = ZERO_FUSED_BATCH;

__device__ __forceinline__ void reduce_adamw_body(const FusedReplicas& reps, int n_rep, int64_t src_off,
                                                  float* __restrict__ master, float* __restrict__ m,
                                                  float* __restrict__ v, uint16_t* __restrict__ param,
                                                  uint16_t* __restrict__ grad_out, int64_t n,
                                                  const AdamScalars& c, const float* __restrict__ clip_scale) {
    const int64_t blk = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t i = blk * kThreads + threadIdx.x;
    if (i >= n) return;
    const float clip = read_clip(clip_scale);
    const bool update = isfinite(clip);
    float p = 0.0f, mm = 0.0f, vv = 0.0f;
    if (update) {                                // state loads in flight beside the replicas'
        p = zero::dev::ld_stream(master + i);
        mm = zero::dev::ld_stream(m + i);
        vv = zero::dev::ld_stream(v + i);
    }
    float acc = 0.0f;
    zero::dev::for_replicas<kFusedBatch, uint16_t>(reps.p, n_rep, src_off, i, [&](uint16_t x) {
        acc = acc + zero::dev::bf16_to_f32(x);
    });
    const uint16_t g = static_cast<uint16_t>(zero::dev::f32_to_bf16(acc / static_cast<float>(n_rep)));
    if (grad_out != nullptr) zero::dev::st_stream(grad_out + i, g);
    if (!update) return;
    adam_elem(p, mm, vv, zero::dev::bf16_to_f32(g) * clip, c);
    zero::dev::st_stream(master + i, p);
    zero::dev::st_stream(m + i, mm);
    zero::dev::st_stream(v + i, vv);
    zero::dev::st_stream(param + i, static_cast<uint16_t>(zero::dev::f32_to_bf16(p)));
}

__global__ __launch_bounds__(kThreads) void reduce_adamw_kernel(FusedReplicas reps, int n_rep,
                                                                int64_t src_off,
                                                                float* __restrict__ master,
                                                                float* __restrict__ m,
                                                                float* __restrict__ v,
                                                                uint16_t* __restrict__ param,
                                                                uint16_t* __restrict__ grad_out,
                                                                int64_t n, AdamScalars c,
                                                                const float* __restrict__ clip_scale) {
    reduce_adamw_body(reps, n_rep, src_off, master, m, v, param, grad_out, n, c, clip_scale);
}

// The one-pass form with the step's scalars read from a schedule's state.
__global__ __launch_bounds__(kThreads) void reduce_adamw_sched_kernel(FusedReplicas reps, int n_rep,
                                                                      int64_t src_off,
                                                                      float* __restrict__ master,
                                                                      float* __restrict__ m,
                                                                      float* __restrict__ v,
                                                                      uint16_t* __restrict__ param,
                                                                      uint16_t* __restrict__ grad_out,
                                                                      int64_t n,
                                                                      const AdamState* __restrict__ state,
                                                                      const float* __restrict__ clip_scale) {
    reduce_adamw_body(reps, n_rep, src_off, master, m, v, param, grad_out, n, state->next, clip_scale);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t blocks_for(int64_t items) {
    const int64_t blocks = (items + kThreads - 1) / kThreads;
    return blocks < 1 ? 1 : blocks;
}

// The checks every multi-tensor call makes on its list (n_tensors > 0).
zero_status check_mt_list(float* const* masters, float* const* exp_avgs, float* const* exp_avg_sqs,
                          const uint16_t* const* grads, uint16_t* const* params_out,
                          const int64_t* numels, int32_t n_tensors, const char* who) {
    using zero::fail;
    const std::string w(who);
    if (!masters || !exp_avgs || !exp_avg_sqs || !grads || !params_out || !numels)
        return fail(ZERO_EINVAL, w + ": NULL array of pointers");
    for (int32_t t = 0; t < n_tensors; ++t) {
        const int64_t n = numels[t];
        if (n < 0) return fail(ZERO_EINVAL, w + ": numel < 0 for tensor " + std::to_string(t));
        if (n == 0) continue;
        if (!masters[t] || !exp_avgs[t] || !exp_avg_sqs[t] || !grads[t] || !params_out[t])
            return fail(ZERO_EINVAL, w + ": NULL array for tensor " + std::to_string(t));
        const size_t fb = static_cast<size_t>(n) * 4, hb = static_cast<size_t>(n) * 2;
        const zero::Span wr[] = {{masters[t], fb, "master"}, {exp_avgs[t], fb, "exp_avg"},
                                 {exp_avg_sqs[t], fb, "exp_avg_sq"}, {params_out[t], hb, "param"}};
        const zero::Span rd[] = {{grads[t], hb, "grad"}};
        const std::string clash = zero::first_overlap(wr, 4, rd, 1);
        if (!clash.empty()) return fail(ZERO_EINVAL, w + ": " + clash + " of tensor " + std::to_string(t));
        if ((n + kMtChunk - 1) / kMtChunk > 0x7FFFFFFF)
            return fail(ZERO_ERANGE, w + ": tensor " + std::to_string(t) + " too large");
    }
    return ZERO_OK;
}

}  // namespace

namespace {

// The flat update's argument checks (n > 0): no NULL array, no written array
// overlapping another array of the call.
zero_status check_flat(float* master, float* exp_avg, float* exp_avg_sq, const uint16_t* grad,
                       uint16_t* param_out, int64_t n, const char* who) {
    using zero::fail;
    if (!master || !exp_avg || !exp_avg_sq || !grad || !param_out)
        return fail(ZERO_EINVAL, std::string(who) + ": NULL array");
    const size_t fbytes = static_cast<size_t>(n) * 4, hbytes = static_cast<size_t>(n) * 2;
    const zero::Span wr[] = {{master, fbytes, "master"}, {exp_avg, fbytes, "exp_avg"},
                             {exp_avg_sq, fbytes, "exp_avg_sq"}, {param_out, hbytes, "param_out"}};
    const zero::Span rd[] = {{grad, hbytes, "grad"}};
    const std::string clash = zero::first_overlap(wr, 4, rd, 1);
    if (!clash.empty()) return fail(ZERO_EINVAL, std::string(who) + ": " + clash);
    return ZERO_OK;
}

// The flat update's launch shape (n > 0): one lane group per lane, the whole
// shard in one dispatch. A grid dimension holds fewer than 2^32 work-items, so
// a larger shard (Llama-3-70B's rank: 8.8e9 elements) takes a grid of up to
// kMaxRow workgroups per row and as many rows as it needs, at most rows - 1
// workgroups past the shard's end. `vec` tells whether every pointer is
// aligned for kEpt elements per lane.
zero_status flat_grid(float* master, float* exp_avg, float* exp_avg_sq, const uint16_t* grad,
                      uint16_t* param_out, int64_t n, dim3* grid, bool* vec, const char* who) {
    constexpr int64_t kMaxRow = (int64_t(1) << 32) / kThreads - 1;
    *vec = kEpt > 1 && aligned(master, 4 * kEpt) && aligned(exp_avg, 4 * kEpt) &&
           aligned(exp_avg_sq, 4 * kEpt) && aligned(grad, 2 * kEpt) && aligned(param_out, 2 * kEpt);
    const int ept = *vec ? kEpt : 1;
    int64_t blocks = blocks_for(n / ept + (n % ept ? 1 : 0));
    if (kPersistPerCu > 0) {
        const int64_t cap = static_cast<int64_t>(kPersistPerCu) * zero::device_cu_count();
        if (blocks > cap) blocks = cap;
    }
    const int64_t rows = (blocks + kMaxRow - 1) / kMaxRow;
    if (rows > 0x7FFFFFFF) return zero::fail(ZERO_ERANGE, std::string(who) + ": n too large for one dispatch");
    *grid = dim3(static_cast<unsigned>((blocks + rows - 1) / rows), static_cast<unsigned>(rows));
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_shard_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                             const uint16_t* grad, uint16_t* param_out, int64_t n,
                                             int64_t step, double lr, double beta1, double beta2,
                                             double eps, double weight_decay,
                                             const float* clip_scale, hipStream_t stream) {
    using zero::fail;
    static const char* const who = "zero_shard_adamw_step";
    zero::clear_error();
    if (n < 0) return fail(ZERO_EINVAL, "zero_shard_adamw_step: n < 0");
    zero_status st = zero::adam::check_hyper(step, lr, beta1, beta2, eps, weight_decay, who);
    if (st != ZERO_OK) return st;
    if (n == 0) return ZERO_OK;
    st = check_flat(master, exp_avg, exp_avg_sq, grad, param_out, n, who);
    if (st != ZERO_OK) return st;
    AdamScalars c;
    st = zero::adam::step_scalars(step, lr, beta1, beta2, weight_decay, eps, &c, who);
    if (st != ZERO_OK) return st;
    dim3 grid;
    bool vec = false;
    st = flat_grid(master, exp_avg, exp_avg_sq, grad, param_out, n, &grid, &vec, who);
    if (st != ZERO_OK) return st;
    if (vec)
        hipLaunchKernelGGL(adamw_kernel<kEpt>, grid, dim3(kThreads), 0, stream, master, exp_avg,
                           exp_avg_sq, grad, param_out, n, c, clip_scale);
    else
        hipLaunchKernelGGL(adamw_kernel<1>, grid, dim3(kThreads), 0, stream, master, exp_avg,
                           exp_avg_sq, grad, param_out, n, c, clip_scale);
    return zero::check_hip(hipGetLastError(), "zero_shard_adamw_step launch");
}

// ------------------------------------------------------------ step schedule

struct zero_adamw_schedule {
    int device = -1;
    void* mem = nullptr;               // the state, then the table
    AdamState* state = nullptr;
    const AdamScalars* table = nullptr;
    int64_t length = 0;
};

extern "C" zero_status zero_adamw_step_scalars(int64_t step, double lr, double beta1, double beta2,
                                               double eps, double weight_decay, float* out) {
    static const char* const who = "zero_adamw_step_scalars";
    zero::clear_error();
    if (out == nullptr) return zero::fail(ZERO_EINVAL, "zero_adamw_step_scalars: NULL out");
    zero_status st = zero::adam::check_hyper(step, lr, beta1, beta2, eps, weight_decay, who);
    if (st != ZERO_OK) return st;
    AdamScalars c;
    st = zero::adam::step_scalars(step, lr, beta1, beta2, weight_decay, eps, &c, who);
    if (st != ZERO_OK) return st;
    const float v[8] = {c.beta1, c.one_minus_beta1, c.beta2, c.one_minus_beta2, c.eps, c.step_size,
                        c.sqrt_bc2, c.decay};
    for (int k = 0; k < 8; ++k) out[k] = v[k];
    return ZERO_OK;
}

extern "C" zero_status zero_adamw_schedule_create(const double* lr, int64_t n_lr, double beta1,
                                                  double beta2, double eps, double weight_decay,
                                                  int64_t first_step, zero_adamw_schedule** out) {
    using zero::fail;
    static const char* const who = "zero_adamw_schedule_create";
    zero::clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "zero_adamw_schedule_create: NULL out");
    *out = nullptr;
    if (first_step < 1) return fail(ZERO_EINVAL, "zero_adamw_schedule_create: first_step must be >= 1");
    std::vector<AdamScalars> table;
    zero_adamw_schedule* sch = nullptr;
    try {
        const zero_status cs = zero::adam::schedule_table(lr, n_lr, beta1, beta2, eps, weight_decay, &table, who);
        if (cs != ZERO_OK) return cs;
        sch = new zero_adamw_schedule;
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_adamw_schedule_create: host allocation failed");
    }
    sch->length = static_cast<int64_t>(table.size());
    AdamState state{};
    state.applied = first_step - 1;
    state.next = table[static_cast<size_t>((first_step < sch->length ? first_step : sch->length) - 1)];
    zero_status st = zero::check_hip(hipGetDevice(&sch->device), who);
    const size_t table_bytes = table.size() * sizeof(AdamScalars);
    if (st == ZERO_OK) st = zero::check_hip(hipMalloc(&sch->mem, 256 + table_bytes), who);
    if (st == ZERO_OK) {
        sch->state = static_cast<AdamState*>(sch->mem);
        sch->table = reinterpret_cast<const AdamScalars*>(static_cast<char*>(sch->mem) + 256);
        st = zero::check_hip(hipMemcpy(sch->state, &state, sizeof(state), hipMemcpyHostToDevice), who);
    }
    if (st == ZERO_OK)
        st = zero::check_hip(hipMemcpy(const_cast<AdamScalars*>(sch->table), table.data(), table_bytes,
                                       hipMemcpyHostToDevice), who);
    if (st != ZERO_OK) {
        if (sch->mem) (void)hipFree(sch->mem);
        delete sch;
        return st;
    }
    *out = sch;
    return ZERO_OK;
}

extern "C" void zero_adamw_schedule_free(zero_adamw_schedule* schedule) {
    if (!schedule) return;
    if (schedule->mem) (void)hipFree(schedule->mem);
    delete schedule;
}

extern "C" int64_t zero_adamw_schedule_length(const zero_adamw_schedule* schedule) {
    return schedule ? schedule->length : -1;
}

extern "C" zero_status zero_adamw_schedule_applied(const zero_adamw_schedule* schedule, int64_t* applied) {
    zero::clear_error();
    if (schedule == nullptr || applied == nullptr)
        return zero::fail(ZERO_EINVAL, "zero_adamw_schedule_applied: NULL schedule or out");
    AdamState state{};
    const zero_status st = zero::check_hip(hipMemcpy(&state, schedule->state, sizeof(state), hipMemcpyDeviceToHost),
                                           "zero_adamw_schedule_applied");
    if (st == ZERO_OK) *applied = state.applied;
    return st;
}

namespace {

zero_status check_schedule_device(const zero_adamw_schedule* schedule, const char* who) {
    int dev = -1;
    const zero_status st = zero::check_hip(hipGetDevice(&dev), who);
    if (st != ZERO_OK) return st;
    if (dev != schedule->device)
        return zero::fail(ZERO_EINVAL, std::string(who) + ": the schedule lives on device " +
                                           std::to_string(schedule->device) + ", the current device is " +
                                           std::to_string(dev));
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_adamw_schedule_advance(zero_adamw_schedule* schedule, const float* clip_scale,
                                                   hipStream_t stream) {
    static const char* const who = "zero_adamw_schedule_advance";
    zero::clear_error();
    if (schedule == nullptr) return zero::fail(ZERO_EINVAL, "zero_adamw_schedule_advance: NULL schedule");
    const zero_status st = check_schedule_device(schedule, who);
    if (st != ZERO_OK) return st;
    hipLaunchKernelGGL(adamw_advance_kernel, dim3(1), dim3(64), 0, stream, schedule->state, schedule->table,
                       schedule->length, clip_scale);
    return zero::check_hip(hipGetLastError(), "zero_adamw_schedule_advance launch");
}

extern "C" zero_status zero_shard_adamw_step_scheduled(float* master, float* exp_avg, float* exp_avg_sq,
                                                       const uint16_t* grad, uint16_t* param_out, int64_t n,
                                                       const zero_adamw_schedule* schedule,
                                                       const float* clip_scale, hipStream_t stream) {
    using zero::fail;
    static const char* const who = "zero_shard_adamw_step_scheduled";
    zero::clear_error();
    if (schedule == nullptr) return fail(ZERO_EINVAL, "zero_shard_adamw_step_scheduled: NULL schedule");
    if (n < 0) return fail(ZERO_EINVAL, "zero_shard_adamw_step_scheduled: n < 0");
    zero_status st = check_schedule_device(schedule, who);
    if (st != ZERO_OK) return st;
    if (n == 0) return ZERO_OK;
    st = check_flat(master, exp_avg, exp_avg_sq, grad, param_out, n, who);
    if (st != ZERO_OK) return st;
    dim3 grid;
    bool vec = false;
    st = flat_grid(master, exp_avg, exp_avg_sq, grad, param_out, n, &grid, &vec, who);
    if (st != ZERO_OK) return st;
    if (vec)
        hipLaunchKernelGGL(adamw_sched_kernel<kEpt>, grid, dim3(kThreads), 0, stream, master, exp_avg,
                           exp_avg_sq, grad, param_out, n, schedule->state, clip_scale);
    else
        hipLaunchKernelGGL(adamw_sched_kernel<1>, grid, dim3(kThreads), 0, stream, master, exp_avg,
                           exp_avg_sq, grad, param_out, n, schedule->state, clip_scale);
    return zero::check_hip(hipGetLastError(), "zero_shard_adamw_step_scheduled launch");
}

extern "C" zero_status zero_multi_tensor_adamw_step(float* const* masters, float* const* exp_avgs,
                                                    float* const* exp_avg_sqs,
                                                    const uint16_t* const* grads,
                                                    uint16_t* const* params_out,
                                                    const int64_t* numels, int32_t n_tensors,
                                                    int64_t step, double lr, double beta1,
                                                    double beta2, double eps, double weight_decay,
                                                    const float* clip_scale, hipStream_t stream) {
    using zero::fail;
    static const char* const who = "zero_multi_tensor_adamw_step";
    zero::clear_error();
    if (n_tensors < 0) return fail(ZERO_EINVAL, "zero_multi_tensor_adamw_step: n_tensors < 0");
    zero_status st = zero::adam::check_hyper(step, lr, beta1, beta2, eps, weight_decay, who);
    if (st != ZERO_OK) return st;
    if (n_tensors == 0) return ZERO_OK;
    st = check_mt_list(masters, exp_avgs, exp_avg_sqs, grads, params_out, numels, n_tensors, who);
    if (st != ZERO_OK) return st;
    AdamScalars c;
    st = zero::adam::step_scalars(step, lr, beta1, beta2, weight_decay, eps, &c, who);
    if (st != ZERO_OK) return st;
    MtBatch batch{};
    auto flush = [&]() -> zero_status {
        if (batch.count == 0) return ZERO_OK;
        hipLaunchKernelGGL(adamw_multi_kernel, dim3(static_cast<unsigned>(batch.first_block[batch.count])),
                           dim3(kThreads), 0, stream, batch, c, clip_scale);
        batch.count = 0;
        batch.first_block[0] = 0;
        return zero::check_hip(hipGetLastError(), "zero_multi_tensor_adamw_step launch");
    };
    // Largest tensors first: the big ones then share a launch, and the many
    // small ones (biases, norms) share the last, instead of every launch
    // mixing both. Each tensor's update is independent, so the order changes
    // no result; on the 148-tensor GPT-2 list it measured 78 us against 82.
    std::vector<int32_t> order;
    try {
        order.resize(static_cast<size_t>(n_tensors));
        for (int32_t t = 0; t < n_tensors; ++t) order[static_cast<size_t>(t)] = t;
        std::stable_sort(order.begin(), order.end(),
                         [numels](int32_t a, int32_t b) { return numels[a] > numels[b]; });
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_multi_tensor_adamw_step: allocation failed");
    }
    for (const int32_t t : order) {
        const int64_t n = numels[t];
        if (n == 0) continue;
        const int64_t blocks = (n + kMtChunk - 1) / kMtChunk;
        if (int64_t(batch.first_block[batch.count]) + blocks > 0x7FFFFFFF) {   // grid < 2^31 workgroups
            st = flush();
            if (st != ZERO_OK) return st;
        }
        const int i = batch.count;
        batch.p[i] = masters[t];
        batch.m[i] = exp_avgs[t];
        batch.v[i] = exp_avg_sqs[t];
        batch.g[i] = grads[t];
        batch.o[i] = params_out[t];
        batch.n[i] = n;
        batch.first_block[i + 1] = batch.first_block[i] + static_cast<int32_t>(blocks);
        batch.count = i + 1;
        if (batch.count == kMtTensors) {
            st = flush();
            if (st != ZERO_OK) return st;
        }
    }
    return flush();
}

// ------------------------------------------------------------ device table

struct zero_mt_table {
    int device = -1;
    void* mem = nullptr;          // descriptors, then the per-workgroup index
    const MtDesc* table = nullptr;
    const uint32_t* index = nullptr;
    int64_t blocks = 0;           // workgroups of one step
};

extern "C" zero_status zero_mt_table_create(float* const* masters, float* const* exp_avgs,
                                            float* const* exp_avg_sqs, const uint16_t* const* grads,
                                            uint16_t* const* params_out, const int64_t* numels,
                                            int32_t n_tensors, zero_mt_table** out) {
    using zero::fail;
    static const char* const who = "zero_mt_table_create";
    zero::clear_error();
    if (!out) return fail(ZERO_EINVAL, "zero_mt_table_create: NULL out");
    *out = nullptr;
    if (n_tensors < 0) return fail(ZERO_EINVAL, "zero_mt_table_create: n_tensors < 0");
    zero_status st = ZERO_OK;
    if (n_tensors > 0) {
        st = check_mt_list(masters, exp_avgs, exp_avg_sqs, grads, params_out, numels, n_tensors, who);
        if (st != ZERO_OK) return st;
    }
    std::vector<MtDesc> descs;
    std::vector<uint32_t> index;
    zero_mt_table* tab = nullptr;
    try {
        int64_t blocks = 0;
        for (int32_t t = 0; t < n_tensors; ++t) {
            const int64_t n = numels[t];
            if (n == 0) continue;
            const int64_t b = (n + kMtChunk - 1) / kMtChunk;
            if (blocks + b > 0x7FFFFFFF)
                return fail(ZERO_ERANGE, "zero_mt_table_create: more than 2^31 workgroups in one list");
            MtDesc d{};
            d.p = masters[t];
            d.m = exp_avgs[t];
            d.v = exp_avg_sqs[t];
            d.g = grads[t];
            d.o = params_out[t];
            d.n = n;
            d.first_block = blocks;
            index.insert(index.end(), static_cast<size_t>(b), static_cast<uint32_t>(descs.size()));
            descs.push_back(d);
            blocks += b;
        }
        if (blocks > 0) index = zero::xcd_major_index(index);
        if (ZERO_MT_DESC_PER_WG && blocks > 0) {      // a descriptor per index entry
            std::vector<MtDesc> per_wg(index.size());
            for (size_t i = 0; i < index.size(); ++i) per_wg[i] = descs[index[i]];
            descs.swap(per_wg);
            index.clear();
        }
        tab = new zero_mt_table;
        tab->blocks = blocks;
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_mt_table_create: host allocation failed");
    }
    if (tab->blocks > 0)          // an empty list needs no device
        st = zero::check_hip(hipGetDevice(&tab->device), "zero_mt_table_create: hipGetDevice");
    if (st == ZERO_OK && tab->blocks > 0) {
        const size_t table_bytes = (descs.size() * sizeof(MtDesc) + 255) / 256 * 256;
        const size_t bytes = table_bytes + index.size() * sizeof(uint32_t);
        st = zero::check_hip(hipMalloc(&tab->mem, bytes), "zero_mt_table_create: hipMalloc");
        if (st == ZERO_OK) {
            tab->table = static_cast<const MtDesc*>(tab->mem);
            tab->index = reinterpret_cast<const uint32_t*>(static_cast<char*>(tab->mem) + table_bytes);
            st = zero::check_hip(hipMemcpy(tab->mem, descs.data(), descs.size() * sizeof(MtDesc),
                                           hipMemcpyHostToDevice), "zero_mt_table_create: hipMemcpy");
        }
        if (st == ZERO_OK && !index.empty())
            st = zero::check_hip(hipMemcpy(const_cast<uint32_t*>(tab->index), index.data(),
                                           index.size() * sizeof(uint32_t), hipMemcpyHostToDevice),
                                 "zero_mt_table_create: hipMemcpy");
    }
    if (st != ZERO_OK) {
        if (tab->mem) (void)hipFree(tab->mem);
        delete tab;
        return st;
    }
    *out = tab;
    return ZERO_OK;
}

extern "C" void zero_mt_table_free(zero_mt_table* table) {
    if (!table) return;
    if (table->mem) (void)hipFree(table->mem);
    delete table;
}

extern "C" int64_t zero_mt_table_blocks(const zero_mt_table* table) {
    return table ? table->blocks : -1;
}

extern "C" zero_status zero_mt_table_adamw_step(const zero_mt_table* table, int64_t step, double lr,
                                                double beta1, double beta2, double eps,
                                                double weight_decay, const float* clip_scale,
                                                hipStream_t stream) {
    using zero::fail;
    static const char* const who = "zero_mt_table_adamw_step";
    zero::clear_error();
    if (!table) return fail(ZERO_EINVAL, "zero_mt_table_adamw_step: NULL table");
    zero_status st = zero::adam::check_hyper(step, lr, beta1, beta2, eps, weight_decay, who);
    if (st != ZERO_OK) return st;
    if (table->blocks == 0) return ZERO_OK;
    int dev = -1;
    st = zero::check_hip(hipGetDevice(&dev), "zero_mt_table_adamw_step: hipGetDevice");
    if (st != ZERO_OK) return st;
    if (dev != table->device)
        return fail(ZERO_EINVAL, "zero_mt_table_adamw_step: the table lives on device " +
                                     std::to_string(table->device) + ", the current device is " +
                                     std::to_string(dev));
    AdamScalars c;
    st = zero::adam::step_scalars(step, lr, beta1, beta2, weight_decay, eps, &c, who);
    if (st != ZERO_OK) return st;
    // A dispatch holds fewer than 2^32 work-items: longer lists take several launches.
    constexpr int64_t kMaxBlocks = zero::kTableLaunchBlocks;
    for (int64_t b0 = 0; b0 < table->blocks; b0 += kMaxBlocks) {
        const int64_t nb = table->blocks - b0 < kMaxBlocks ? table->blocks - b0 : kMaxBlocks;
        const int64_t per = (nb + 7) / 8;
        hipLaunchKernelGGL(adamw_table_kernel, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0,
                           stream, table->table, table->index, b0, per, c, clip_scale);
        st = zero::check_hip(hipGetLastError(), "zero_mt_table_adamw_step launch");
        if (st != ZERO_OK) return st;
    }
    return ZERO_OK;
}

extern "C" zero_status zero_mt_table_adamw_step_scheduled(const zero_mt_table* table,
                                                          const zero_adamw_schedule* schedule,
                                                          const float* clip_scale, hipStream_t stream) {
    using zero::fail;
    static const char* const who = "zero_mt_table_adamw_step_scheduled";
    zero::clear_error();
    if (!table || !schedule) return fail(ZERO_EINVAL, "zero_mt_table_adamw_step_scheduled: NULL table or schedule");
    zero_status st = check_schedule_device(schedule, who);
    if (st != ZERO_OK) return st;
    if (table->blocks == 0) return ZERO_OK;
    if (table->device != schedule->device)
        return fail(ZERO_EINVAL, "zero_mt_table_adamw_step_scheduled: the table lives on device " +
                                     std::to_string(table->device) + ", the schedule on device " +
                                     std::to_string(schedule->device));
    constexpr int64_t kMaxBlocks = zero::kTableLaunchBlocks;
    for (int64_t b0 = 0; b0 < table->blocks; b0 += kMaxBlocks) {
        const int64_t nb = table->blocks - b0 < kMaxBlocks ? table->blocks - b0 : kMaxBlocks;
        const int64_t per = (nb + 7) / 8;
        hipLaunchKernelGGL(adamw_table_sched_kernel, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0,
                           stream, table->table, table->index, b0, per, schedule->state, clip_scale);
        st = zero::check_hip(hipGetLastError(), "zero_mt_table_adamw_step_scheduled launch");
        if (st != ZERO_OK) return st;
    }
    return ZERO_OK;
}

namespace {

// The one-pass reduce and update's window checks.
zero_status fused_check_window(const zero_plan* plan, int32_t rank, const uint16_t* const* replicas,
                               int32_t n_replicas, int64_t begin, int64_t count, const char* who) {
    using zero::fail;
    const std::string w(who);
    if (plan == nullptr || replicas == nullptr) return fail(ZERO_EINVAL, w + ": NULL plan or replicas");
    if (rank < 0 || rank >= plan->n_ranks) return fail(ZERO_EINVAL, w + ": rank out of range");
    if (n_replicas < 1 || n_replicas > ZERO_MAX_REPLICAS)
        return fail(ZERO_EINVAL, w + ": n_replicas must be 1.." + std::to_string(ZERO_MAX_REPLICAS));
    if (begin < 0 || count < 0 || begin > plan->padded || count > plan->padded - begin)
        return fail(ZERO_EINVAL, w + ": window outside [0, P)");
    return ZERO_OK;
}

// Its launch: the window's part of the rank's shard, the replica table, the
// grid (rows of workgroups past 2^32 work-items). `empty` when the window
// misses the shard.
struct FusedCall {
    FusedReplicas table{};
    int64_t n = 0, src_off = 0, at = 0;
    dim3 grid;
    bool empty = true;
};

zero_status fused_prepare(const zero_plan* plan, int32_t rank, const uint16_t* const* replicas,
                          int32_t n_replicas, int64_t begin, int64_t count, float* master, float* exp_avg,
                          float* exp_avg_sq, uint16_t* param_out, uint16_t* shard_grad, const char* who,
                          FusedCall* call) {
    using zero::fail;
    const std::string w(who);
    const int64_t shard_lo = static_cast<int64_t>(rank) * plan->shard;
    const int64_t lo = begin > shard_lo ? begin : shard_lo;
    const int64_t end = begin + count, shard_hi = shard_lo + plan->shard;
    const int64_t hi = end < shard_hi ? end : shard_hi;
    call->empty = lo >= hi;
    if (call->empty) return ZERO_OK;
    if (!master || !exp_avg || !exp_avg_sq || !param_out) return fail(ZERO_EINVAL, w + ": NULL state array");
    for (int32_t k = 0; k < n_replicas; ++k) {
        if (replicas[k] == nullptr) return fail(ZERO_EINVAL, w + ": NULL replica");
        call->table.p[k] = replicas[k];
    }
    const int64_t n = hi - lo, src_off = lo - begin, at = lo - shard_lo;
    const size_t fbytes = static_cast<size_t>(n) * 4, hbytes = static_cast<size_t>(n) * 2;
    const zero::Span wr[] = {{master + at, fbytes, "master"}, {exp_avg + at, fbytes, "exp_avg"},
                             {exp_avg_sq + at, fbytes, "exp_avg_sq"}, {param_out + at, hbytes, "param_out"},
                             {shard_grad != nullptr ? shard_grad + at : nullptr, shard_grad ? hbytes : 0,
                              "shard_grad"}};
    zero::Span rd[ZERO_MAX_REPLICAS];
    for (int32_t k = 0; k < n_replicas; ++k) rd[k] = {replicas[k] + src_off, hbytes, "replica", k};
    const std::string clash = zero::first_overlap(wr, 5, rd, n_replicas);
    if (!clash.empty()) return fail(ZERO_EINVAL, w + ": " + clash);
    constexpr int64_t kMaxRow = (int64_t(1) << 32) / kThreads - 1;
    const int64_t blocks = blocks_for(n);
    const int64_t rows = (blocks + kMaxRow - 1) / kMaxRow;
    call->grid = dim3(static_cast<unsigned>((blocks + rows - 1) / rows), static_cast<unsigned>(rows));
    call->n = n;
    call->src_off = src_off;
    call->at = at;
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_reduce_adamw_step(const zero_plan* plan, int32_t rank,
                                              const uint16_t* const* replicas, int32_t n_replicas,
                                              int64_t begin, int64_t count, float* master,
                                              float* exp_avg, float* exp_avg_sq, uint16_t* param_out,
                                              uint16_t* shard_grad, int64_t step, double lr,
                                              double beta1, double beta2, double eps,
                                              double weight_decay, const float* clip_scale,
                                              hipStream_t stream) {
    static const char* const who = "zero_reduce_adamw_step";
    zero::clear_error();
    zero_status st = fused_check_window(plan, rank, replicas, n_replicas, begin, count, who);
    if (st != ZERO_OK) return st;
    st = zero::adam::check_hyper(step, lr, beta1, beta2, eps, weight_decay, who);
    if (st != ZERO_OK) return st;
    FusedCall call;
    st = fused_prepare(plan, rank, replicas, n_replicas, begin, count, master, exp_avg, exp_avg_sq, param_out,
                       shard_grad, who, &call);
    if (st != ZERO_OK || call.empty) return st;
    AdamScalars c;
    st = zero::adam::step_scalars(step, lr, beta1, beta2, weight_decay, eps, &c, who);
    if (st != ZERO_OK) return st;
    const int64_t at = call.at;
    hipLaunchKernelGGL(reduce_adamw_kernel, call.grid, dim3(kThreads), 0, stream, call.table, n_replicas,
                       call.src_off, master + at, exp_avg + at, exp_avg_sq + at, param_out + at,
                       shard_grad != nullptr ? shard_grad + at : nullptr, call.n, c, clip_scale);
    return zero::check_hip(hipGetLastError(), "zero_reduce_adamw_step launch");
}

extern "C" zero_status zero_reduce_adamw_step_scheduled(const zero_plan* plan, int32_t rank,
                                                        const uint16_t* const* replicas, int32_t n_replicas,
                                                        int64_t begin, int64_t count, float* master,
                                                        float* exp_avg, float* exp_avg_sq,
                                                        uint16_t* param_out, uint16_t* shard_grad,
                                                        const zero_adamw_schedule* schedule,
                                                        const float* clip_scale, hipStream_t stream) {
    static const char* const who = "zero_reduce_adamw_step_scheduled";
    zero::clear_error();
    if (schedule == nullptr) return zero::fail(ZERO_EINVAL, "zero_reduce_adamw_step_scheduled: NULL schedule");
    zero_status st = fused_check_window(plan, rank, replicas, n_replicas, begin, count, who);
    if (st != ZERO_OK) return st;
    st = check_schedule_device(schedule, who);
    if (st != ZERO_OK) return st;
    FusedCall call;
    st = fused_prepare(plan, rank, replicas, n_replicas, begin, count, master, exp_avg, exp_avg_sq, param_out,
                       shard_grad, who, &call);
    if (st != ZERO_OK || call.empty) return st;
    const int64_t at = call.at;
    hipLaunchKernelGGL(reduce_adamw_sched_kernel, call.grid, dim3(kThreads), 0, stream, call.table, n_replicas,
                       call.src_off, master + at, exp_avg + at, exp_avg_sq + at, param_out + at,
                       shard_grad != nullptr ? shard_grad + at : nullptr, call.n, schedule->state, clip_scale);
    return zero::check_hip(hipGetLastError(), "zero_reduce_adamw_step_scheduled launch");
}
