// Launch shape of the bf16 copy kernels (gather and flatten), and the index
// map of their tensor-major form for Shard(0) plans: which rank buffer, and
// where in it, the elements of each lane lie. Shared by the kernels in
// gather.hip and by a host-side check of every wave's store addresses.
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "FSDP-2: Per-Parameter Sharding via
// DTensor (fully_shard)": each tensor is cut along dim 0 into N_d chunks, rank
// r's chunk at the same offset of every rank's coalesced buffer. Element e of a
// tensor whose full chunk holds `chunk` elements lies in rank e / chunk, at
// e % chunk inside that rank's chunk.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace zero {
namespace copy {

constexpr int kThreads = 256;
// One access per lane: ZERO_GATHER_LANE_ELEMS bf16 values (8 = 16 bytes).
#ifndef ZERO_GATHER_LANE_ELEMS
#define ZERO_GATHER_LANE_ELEMS 8
#endif
constexpr int kLane = ZERO_GATHER_LANE_ELEMS;
// Accesses per lane: a workgroup copies kVecs passes of kRow elements, so its
// fixed start-up work (finding its descriptor) is paid once per kChunk.
#ifndef ZERO_GATHER_VECS
#define ZERO_GATHER_VECS 1
#endif
constexpr int kVecs = ZERO_GATHER_VECS;
constexpr int64_t kRow = int64_t(kThreads) * kLane;     // elements per pass
constexpr int64_t kChunk = kRow * kVecs;                // elements per workgroup

// Tensor-major form: tensors of fewer than 2^31 elements (32-bit division),
// plans of at most kMaxRanks ranks (the rank pointers travel in the kernel
// arguments).
constexpr int kMaxRanks = 64;
constexpr int64_t kMaxTensorElems = (int64_t(1) << 31) - 1;
// Plans of at most kCompactRanks ranks whose shards hold fewer than 2^31
// elements use the compact argument table (32-bit chunk offsets).
constexpr int kCompactRanks = 8;

// Shard(0) plans whose tensors all fit the 32-bit division, on at most
// kMaxRanks ranks, take the tensor-major kernel; the others the segment kernels.
inline bool fits_tensor_major(const zero_plan* plan) {
    if (plan->kind != 1 || plan->n_ranks > kMaxRanks || plan->shard <= 0) return false;
    for (const int64_t n : plan->numels)
        if (n > kMaxTensorElems) return false;
    return true;
}

inline bool fits_compact(const zero_plan* plan) {
    return plan->n_ranks <= kCompactRanks && plan->shard < (int64_t(1) << 31);
}

// Where a workgroup's first element e0 lies: rank r0 = e0 / chunk, and its
// offset local0 = e0 - r0 * chunk inside rank r0's chunk.
struct WorkgroupStart {
    int32_t r0;
    int64_t local0;
};
__host__ __device__ inline WorkgroupStart workgroup_start(int64_t e0, int64_t chunk) {
    const uint32_t q0 = static_cast<uint32_t>(e0) / static_cast<uint32_t>(chunk);
    return {static_cast<int32_t>(q0), e0 - static_cast<int64_t>(q0) * chunk};
}

// The lane whose first element is e0 + j (j = its offset in the workgroup):
// the rank buffer holding that element and its offset inside the rank's chunk.
// "big" is the workgroup-uniform choice chunk >= kChunk: a workgroup's
// elements then lie in rank r0 or r0 + 1 (local0 + j < chunk + kChunk <= 2 *
// chunk), found by one comparison; otherwise by a 32-bit division per lane
// (local0 + j < chunk + kChunk < 2 * kChunk).
struct LanePlace {
    int32_t rank;
    int64_t within;
};
__host__ __device__ inline LanePlace lane_place(const WorkgroupStart& ws, int64_t chunk, int64_t j,
                                                bool big) {
    if (big) {
        const int64_t local = ws.local0 + j;
        const bool next = local >= chunk;
        return {ws.r0 + (next ? 1 : 0), next ? local - chunk : local};
    }
    const uint32_t lj = static_cast<uint32_t>(ws.local0 + j);
    const uint32_t c32 = static_cast<uint32_t>(chunk);
    const uint32_t q = lj / c32;
    return {ws.r0 + static_cast<int32_t>(q), static_cast<int64_t>(lj - q * c32)};
}

// The lane copies its kLane elements with one vector access when they all lie
// in the tensor and in the one rank chunk, and both addresses are aligned to
// the access; element by element otherwise.
__host__ __device__ inline bool lane_whole(int64_t e, int64_t numel, int64_t within, int64_t chunk,
                                           uintptr_t buf_addr, uintptr_t tensor_addr) {
    return e + kLane <= numel && within + kLane <= chunk &&
           ((buf_addr | tensor_addr) & static_cast<uintptr_t>(2 * kLane - 1)) == 0;
}

}  // namespace copy
}  // namespace zero
