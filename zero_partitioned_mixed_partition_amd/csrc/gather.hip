// Gather of bf16 parameter shards into per-tensor parameters, and its inverse,
// the flatten of per-tensor buffers into the padded flat buffer (gfx950).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "Execution Flow for ZeRO-1", step 4:
// the all-gather rebuilds the complete 16-bit parameters from every rank's
// shard; section "FSDP-1": the shards are equal chunks of one flat buffer, so
// each tensor is a slice of the shards' concatenation. The plan lists that
// slice as segments (tensor, offset in tensor, shard, offset in shard,
// length); this kernel copies every segment.
//
// Memory: 2 bytes read and 2 written per parameter. The segment table travels
// in the kernel arguments, kSegs segments per launch (no device-side table,
// no host-to-device copy, nothing allocated): workgroup b finds its segment by
// a binary search over the per-segment workgroup prefix, then copies a chunk
// of kChunk elements, one access per lane (16 bytes by default) with
// non-temporal hints when source and destination are co-aligned to the access
// width, element by element otherwise.
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "device_common.hpp"
#include "internal.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kSegs = 96;                       // segments per launch (kernarg ~3.1 KB of the 4 KB limit)
// One access per lane: ZERO_GATHER_LANE_ELEMS bf16 values (8 = 16 bytes).
#ifndef ZERO_GATHER_LANE_ELEMS
#define ZERO_GATHER_LANE_ELEMS 8
#endif
constexpr int kLane = ZERO_GATHER_LANE_ELEMS;
constexpr int64_t kChunk = int64_t(kThreads) * kLane;   // elements per workgroup

template <int E> struct LaneBits;
template <> struct LaneBits<8> { typedef zero::dev::u32x4 T; };
template <> struct LaneBits<4> { typedef zero::dev::u32x2 T; };
template <> struct LaneBits<2> { typedef uint32_t T; };

struct SegBatch {
    const uint16_t* src[kSegs];
    uint16_t* dst[kSegs];
    int64_t len[kSegs];
    int64_t first_block[kSegs + 1];   // workgroups [first_block[s], first_block[s+1]) copy segment s
    int32_t n;
};

__global__ __launch_bounds__(kThreads) void gather_kernel(SegBatch b) {
    typedef typename LaneBits<kLane>::T V;
    const int64_t blk = blockIdx.x;
    int lo = 0, hi = b.n - 1;                         // find s with first_block[s] <= blk < first_block[s+1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (b.first_block[mid] <= blk) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const int64_t start = (blk - b.first_block[s]) * kChunk;
    const int64_t len = b.len[s] - start < kChunk ? b.len[s] - start : kChunk;
    uint16_t* dst = b.dst[s] + start;
    if (b.src[s] == nullptr) {                        // padding: fill with +0
        const int64_t i = threadIdx.x;
        if (i * kLane + kLane <= len && (reinterpret_cast<uintptr_t>(dst) & (2 * kLane - 1)) == 0) {
            zero::dev::st_stream(reinterpret_cast<V*>(dst) + i, V{});
        } else {
            for (int64_t e = i * kLane; e < len && e < i * kLane + kLane; ++e) dst[e] = 0;
        }
        return;
    }
    const uint16_t* src = b.src[s] + start;
    constexpr uintptr_t kBytes = 2 * kLane;
    const uintptr_t sa = reinterpret_cast<uintptr_t>(src), da = reinterpret_cast<uintptr_t>(dst);
    if (((sa ^ da) & (kBytes - 1)) == 0) {
        // Co-aligned: element head up to the access boundary, vector body, element tail.
        int64_t head = static_cast<int64_t>(((kBytes - (da & (kBytes - 1))) & (kBytes - 1)) / 2u);
        if (head > len) head = len;
        if (threadIdx.x < head) dst[threadIdx.x] = src[threadIdx.x];
        const int64_t body = (len - head) / kLane;
        const V* sv = reinterpret_cast<const V*>(src + head);
        V* dv = reinterpret_cast<V*>(dst + head);
        const int64_t i = threadIdx.x;
        if (i < body) zero::dev::st_stream(dv + i, zero::dev::ld_stream(sv + i));
        const int64_t t = head + body * kLane + threadIdx.x;
        if (t < len) dst[t] = src[t];
    } else {
        for (int64_t i = threadIdx.x; i < len; i += kThreads) dst[i] = src[i];
    }
}

}  // namespace

namespace {

// Launches one segment-copy kernel per kSegs segments. Each piece is
// (src, dst, len); a NULL src fills dst with zeros.
struct Piece {
    const uint16_t* src;
    uint16_t* dst;
    int64_t len;
};

zero_status launch_pieces(const std::vector<Piece>& pieces, hipStream_t stream, const char* who) {
    SegBatch batch{};
    auto flush = [&]() -> zero_status {
        if (batch.n == 0) return ZERO_OK;
        const int64_t blocks = batch.first_block[batch.n];
        hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                           stream, batch);
        batch.n = 0;
        batch.first_block[0] = 0;
        return zero::check_hip(hipGetLastError(), who);
    };
    for (const Piece& pc : pieces) {
        if (pc.len <= 0) continue;
        const int64_t chunks = (pc.len + kChunk - 1) / kChunk;
        if (batch.first_block[batch.n] + chunks > 0x7FFFFFFF) {   // one grid < 2^31 workgroups
            const zero_status st = flush();
            if (st != ZERO_OK) return st;
        }
        if (chunks > 0x7FFFFFFF) return zero::fail(ZERO_ERANGE, std::string(who) + ": segment too long");
        const int i = batch.n;
        batch.src[i] = pc.src;
        batch.dst[i] = pc.dst;
        batch.len[i] = pc.len;
        batch.first_block[i + 1] = batch.first_block[i] + chunks;
        batch.n = i + 1;
        if (batch.n == kSegs) {
            const zero_status st = flush();
            if (st != ZERO_OK) return st;
        }
    }
    return flush();
}

zero_status check_tensors(const zero_plan* plan, const uint16_t* const* tensors, const char* who) {
    if (!plan->numels.empty() && tensors == nullptr)
        return zero::fail(ZERO_EINVAL, std::string(who) + ": NULL tensors");
    for (size_t t = 0; t < plan->numels.size(); ++t)
        if (plan->numels[t] > 0 && tensors[t] == nullptr)
            return zero::fail(ZERO_EINVAL, std::string(who) + ": NULL tensor " + std::to_string(t));
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_gather_params(const zero_plan* plan, const uint16_t* const* shards,
                                          uint16_t* const* tensors, hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (plan == nullptr || shards == nullptr)
        return fail(ZERO_EINVAL, "zero_gather_params: NULL plan or shards");
    zero_status st = check_tensors(plan, tensors, "zero_gather_params");
    if (st != ZERO_OK) return st;
    for (int32_t r = 0; r < plan->n_ranks; ++r)
        if (plan->shard > 0 && shards[r] == nullptr)
            return fail(ZERO_EINVAL, "zero_gather_params: NULL shard " + std::to_string(r));
    std::vector<Piece> pieces;
    pieces.reserve(plan->all.size());
    for (const zero_segment& seg : plan->all)
        pieces.push_back({shards[seg.rank] + seg.shard_offset, tensors[seg.tensor] + seg.tensor_offset,
                          seg.length});
    return launch_pieces(pieces, stream, "zero_gather_params launch");
}

extern "C" zero_status zero_flatten_params(const zero_plan* plan, const uint16_t* const* tensors,
                                           uint16_t* flat, hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (plan == nullptr) return fail(ZERO_EINVAL, "zero_flatten_params: NULL plan");
    if (plan->padded > 0 && flat == nullptr) return fail(ZERO_EINVAL, "zero_flatten_params: NULL flat");
    zero_status st = check_tensors(plan, tensors, "zero_flatten_params");
    if (st != ZERO_OK) return st;
    // Every segment, in flat order, copied to its place; every gap between
    // segments (and after the last) filled with zeros.
    std::vector<Piece> pieces;
    pieces.reserve(2 * plan->all.size() + 1);
    int64_t pos = 0;
    for (const zero_segment& seg : plan->all) {
        const int64_t at = static_cast<int64_t>(seg.rank) * plan->shard + seg.shard_offset;
        if (at > pos) pieces.push_back({nullptr, flat + pos, at - pos});
        pieces.push_back({tensors[seg.tensor] + seg.tensor_offset, flat + at, seg.length});
        pos = at + seg.length;
    }
    if (plan->padded > pos) pieces.push_back({nullptr, flat + pos, plan->padded - pos});
    return launch_pieces(pieces, stream, "zero_flatten_params launch");
}
