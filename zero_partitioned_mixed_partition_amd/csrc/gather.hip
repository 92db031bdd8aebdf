// Gather of bf16 parameter shards into per-tensor parameters, and its inverse,
// the flatten of per-tensor buffers into the padded flat buffer (gfx950).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "Execution Flow for ZeRO-1", step 4:
// the all-gather rebuilds the complete 16-bit parameters from every rank's
// shard; section "FSDP-1": the shards are equal chunks of one flat buffer, so
// each tensor is a slice of the shards' concatenation. The plan lists that
// slice as segments (tensor, offset in tensor, shard, offset in shard,
// length). Section "FSDP-2: Per-Parameter Sharding via DTensor": with
// per-parameter Shard(0) placement, each tensor is its ranks' dim-0 chunks
// stacked in rank order.
//
// Memory: 2 bytes read and 2 written per parameter. Three kernels, all copying
// kChunk elements per workgroup, one access per lane (16 bytes by default)
// when source and destination allow it, element by element otherwise:
//   gather_kernel         one descriptor per plan segment (also the flatten),
//                         tables in the kernel arguments;
//   gather_tensor_kernel  one descriptor per tensor, tables in the kernel
//                         arguments; the rank of an element is found by
//                         arithmetic. A Shard(0) plan has about N_d segments
//                         per tensor, so this needs N_d times fewer
//                         descriptors, and launches, than the segment form;
//   copy_table_kernel     for fixed buffers: every piece described once in
//                         device memory (a copy table), with a descriptor
//                         index per workgroup, in one launch.
// The call forms allocate nothing and copy nothing to the device; a copy table
// does both once, at creation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "device_common.hpp"
#include "internal.hpp"
#include "pieces.hpp"
#include "tensor_major.hpp"

namespace {

using zero::copy::kChunk;
using zero::copy::kLane;
using zero::copy::kThreads;
using zero::copy::kVecs;
constexpr int kSegs = 160;                      // segments per launch (kernarg ~3.8 KB of the 4 KB limit)
constexpr int64_t kMaxPiece = int64_t(1) << 30; // longer pieces are split: lengths fit 32 bits

template <int E> struct LaneBits;
template <> struct LaneBits<8> { typedef zero::dev::u32x4 T; };
template <> struct LaneBits<4> { typedef zero::dev::u32x2 T; };
template <> struct LaneBits<2> { typedef uint32_t T; };

struct SegBatch {
    const uint16_t* src[kSegs];
    uint16_t* dst[kSegs];
    int32_t len[kSegs];               // elements, at most kMaxPiece
    int32_t first_block[kSegs + 1];   // workgroups [first_block[s], first_block[s+1]) copy segment s
    int32_t n;
};
static_assert(sizeof(SegBatch) <= 4096, "kernel arguments are limited to 4 KB");

// One workgroup's chunk of a piece: len (<= kChunk) elements from src to dst,
// or zeros when src is NULL.
__device__ __forceinline__ void copy_chunk(const uint16_t* src, uint16_t* dst, int64_t len) {
    typedef typename LaneBits<kLane>::T V;
    if (src == nullptr) {                             // padding: fill with +0
        const bool aligned = (reinterpret_cast<uintptr_t>(dst) & (2 * kLane - 1)) == 0;
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {
            const int64_t i = int64_t(v) * kThreads + threadIdx.x;
            if (aligned && i * kLane + kLane <= len) {
                zero::dev::st_stream(reinterpret_cast<V*>(dst) + i, V{});
            } else {
                for (int64_t e = i * kLane; e < len && e < i * kLane + kLane; ++e) dst[e] = 0;
            }
        }
        return;
    }
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
        V vals[kVecs];
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {            // all loads first, then all stores
            const int64_t i = int64_t(v) * kThreads + threadIdx.x;
            if (i < body) vals[v] = zero::dev::ld_stream(sv + i);
        }
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {
            const int64_t i = int64_t(v) * kThreads + threadIdx.x;
            if (i < body) zero::dev::st_stream(dv + i, vals[v]);
        }
        const int64_t t = head + body * kLane + threadIdx.x;
        if (t < len) dst[t] = src[t];
    } else {
        for (int64_t i = threadIdx.x; i < len; i += kThreads) dst[i] = src[i];
    }
}

__global__ __launch_bounds__(kThreads) void gather_kernel(SegBatch b) {
    const int64_t blk = blockIdx.x;
    int lo = 0, hi = b.n - 1;                         // find s with first_block[s] <= blk < first_block[s+1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (b.first_block[mid] <= blk) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const int64_t start = (blk - b.first_block[s]) * kChunk;
    const int64_t seg_len = b.len[s];
    const int64_t len = seg_len - start < kChunk ? seg_len - start : kChunk;
    copy_chunk(b.src[s] != nullptr ? b.src[s] + start : nullptr, b.dst[s] + start, len);
}

// Device-resident form for fixed buffers: one 32-byte descriptor per piece and,
// per workgroup, the index of its descriptor, so a workgroup finds its piece
// with two dependent scalar loads and every piece of a plan (a Shard(0) plan
// has about N_d per tensor) goes out in one launch.
using zero::copy::PieceDesc;

__global__ __launch_bounds__(kThreads) void copy_table_kernel(const PieceDesc* __restrict__ table,
                                                              const uint32_t* __restrict__ index,
                                                              int64_t blk0, int64_t per) {
    const int64_t blk = blk0 + static_cast<int64_t>(blockIdx.x);
    const PieceDesc d = table[index[zero::dev::xcd_major_entry(blk0, per)]];
    const int64_t start = (blk - d.first_block) * kChunk;
    const int64_t len = d.len - start < kChunk ? d.len - start : kChunk;
    copy_chunk(d.src != nullptr ? d.src + start : nullptr, d.dst + start, len);
}

// Tensor-major gather for Shard(0) plans: one descriptor per tensor instead of
// one per segment. Element e of tensor t lies in rank r = e / chunk_t
// (chunk_t = rows per chunk * elements per row) and is read from shards[r] +
// off_t + (e - r*chunk_t), off_t being the chunk's start in every rank's
// coalesced buffer (the index map is in tensor_major.hpp). A workgroup copies
// kChunk elements of one tensor: it finds the rank of its first element once,
// and when chunk_t >= kChunk its lanes lie in that rank or the next, two
// workgroup-uniform shard pointers. Smaller chunks take a per-lane division.
//
// Stores: the gather writes one tensor, so each wave's stores are one
// contiguous run (st_stream). The flatten writes rank buffers, which lie S
// elements apart, and one wave can span a chunk boundary: with large chunks
// each store takes its own rank's chunk start as the buffer base (st_stream_at,
// offsets below 2 * chunk_t < 2^32 bytes), with small chunks a lane's rank is
// its own and the stores are global ones (st_stream_any).
//
// The descriptors travel in the kernel arguments (4 KB). The wide table has
// room for 64 rank pointers and 64-bit chunk offsets (127 tensors per launch);
// plans with at most 8 ranks and shards under 2^31 elements use the compact
// table, 8 rank pointers and 32-bit offsets, which fits 167 tensors: GPT-2
// small's 148 in one launch instead of two.
template <int kR, typename Off>
struct TensorBatch {
    using OffT = Off;
    static constexpr int kRanks = kR;
    static constexpr int kTens = (4096 - 8 * kR - 8) / (8 + static_cast<int>(sizeof(Off)) + 12);
    uint16_t* shards[kR];         // rank buffers (read by the gather, written by the flatten)
    uint16_t* dst[kTens];         // tensors (written by the gather, read by the flatten)
    Off off[kTens];               // the chunk's start in a rank's coalesced buffer
    int32_t numel[kTens];
    int32_t chunk[kTens];
    int32_t first_block[kTens + 1];
    int32_t n;
};
using WideBatch = TensorBatch<zero::copy::kMaxRanks, int64_t>;
using CompactBatch = TensorBatch<zero::copy::kCompactRanks, int32_t>;
static_assert(sizeof(WideBatch) <= 4096 && sizeof(CompactBatch) <= 4096,
              "kernel arguments are limited to 4 KB");
static_assert(WideBatch::kTens >= 120 && CompactBatch::kTens >= 160, "table capacities");

// kScatter = false: the gather (rank buffers -> tensors); true: the flatten
// (tensors -> rank buffers), the same index map copied the other way.
template <bool kScatter>
__device__ __forceinline__ void copy_elem(uint16_t* tens, uint16_t* buf) {
    if (kScatter) *buf = *tens; else *tens = *buf;
}

template <bool kScatter, class Batch>
__global__ __launch_bounds__(kThreads) void gather_tensor_kernel(Batch b) {
    typedef typename LaneBits<kLane>::T V;
    using zero::copy::LanePlace;
    using zero::copy::lane_place;
    using zero::copy::lane_whole;
    const int64_t blk = blockIdx.x;
    int lo = 0, hi = b.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (b.first_block[mid] <= blk) lo = mid; else hi = mid - 1;
    }
    const int t = lo;
    const int64_t e0 = (blk - b.first_block[t]) * kChunk;        // workgroup's first element
    const int64_t numel = b.numel[t], chunk = b.chunk[t];
    const int64_t soff = b.off[t];
    zero::copy::WorkgroupStart ws = zero::copy::workgroup_start(e0, chunk);
    ws.r0 = __builtin_amdgcn_readfirstlane(ws.r0);
    uint16_t* dst = b.dst[t];
    if (chunk >= kChunk) {
        // rank r0, or r0 + 1 past the boundary
        uint16_t* p0 = b.shards[ws.r0] + soff;
        uint16_t* p1 = (ws.r0 + 1 < Batch::kRanks ? b.shards[ws.r0 + 1] : b.shards[ws.r0]) + soff;
        V vals[kVecs];
        bool fast[kVecs];
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {            // all loads first, then all stores
            const int64_t j = (int64_t(v) * kThreads + threadIdx.x) * kLane;
            const int64_t e = e0 + j;
            const LanePlace pl = lane_place(ws, chunk, j, true);
            const uint16_t* buf = (pl.rank != ws.r0 ? p1 : p0) + pl.within;
            fast[v] = lane_whole(e, numel, pl.within, chunk, reinterpret_cast<uintptr_t>(buf),
                                 reinterpret_cast<uintptr_t>(dst + e));
            if (fast[v]) vals[v] = zero::dev::ld_stream(reinterpret_cast<const V*>(kScatter ? dst + e : buf));
        }
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {
            const int64_t j = (int64_t(v) * kThreads + threadIdx.x) * kLane;
            const int64_t e = e0 + j;
            const LanePlace pl = lane_place(ws, chunk, j, true);
            if (fast[v]) {
                if (kScatter) {
                    const uint32_t off = static_cast<uint32_t>(pl.within * 2);
                    if (pl.rank != ws.r0)
                        zero::dev::st_stream_at(p1, off, vals[v]);
                    else
                        zero::dev::st_stream_at(p0, off, vals[v]);
                } else {
                    zero::dev::st_stream(reinterpret_cast<V*>(dst + e), vals[v]);
                }
                continue;
            }
            // Straddles the boundary, misaligned, or the tensor's tail.
            const int64_t local = ws.local0 + j;
            for (int k = 0; k < kLane && e + k < numel; ++k) {
                const int64_t lk = local + k;
                copy_elem<kScatter>(dst + e + k, lk < chunk ? p0 + lk : p1 + (lk - chunk));
            }
        }
        return;
    }
    // Small chunks: a lane's rank by a 32-bit division; a lane's elements may
    // lie in several ranks.
    const uint32_t c32 = static_cast<uint32_t>(chunk);
    for (int v = 0; v < kVecs; ++v) {
        const int64_t j = (int64_t(v) * kThreads + threadIdx.x) * kLane;
        const int64_t e = e0 + j;
        if (e >= numel) break;
        const LanePlace pl = lane_place(ws, chunk, j, false);
        uint16_t* buf = b.shards[pl.rank] + soff + pl.within;
        if (lane_whole(e, numel, pl.within, chunk, reinterpret_cast<uintptr_t>(buf),
                       reinterpret_cast<uintptr_t>(dst + e))) {
            if (kScatter)
                zero::dev::st_stream_any(reinterpret_cast<V*>(buf), zero::dev::ld_stream(reinterpret_cast<const V*>(dst + e)));
            else
                zero::dev::st_stream(reinterpret_cast<V*>(dst + e), zero::dev::ld_stream(reinterpret_cast<const V*>(buf)));
            continue;
        }
        const uint32_t lj = static_cast<uint32_t>(ws.local0 + j);
        for (int k = 0; k < kLane && e + k < numel; ++k) {
            const uint32_t lk = lj + static_cast<uint32_t>(k);
            const uint32_t qk = lk / c32;
            copy_elem<kScatter>(dst + e + k, b.shards[ws.r0 + static_cast<int>(qk)] + soff + (lk - qk * c32));
        }
    }
}

}  // namespace

namespace {

// Launches one segment-copy kernel per kSegs segments. Each piece is
// (src, dst, len); a NULL src fills dst with zeros.
using zero::copy::Piece;

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
    for (const Piece& whole : pieces) {
        for (int64_t at = 0; at < whole.len; at += kMaxPiece) {
            const int64_t len = whole.len - at < kMaxPiece ? whole.len - at : kMaxPiece;
            const int64_t chunks = (len + kChunk - 1) / kChunk;
            if (int64_t(batch.first_block[batch.n]) + chunks > 0x7FFFFFFF) {   // grid < 2^31 workgroups
                const zero_status st = flush();
                if (st != ZERO_OK) return st;
            }
            const int i = batch.n;
            batch.src[i] = whole.src != nullptr ? whole.src + at : nullptr;
            batch.dst[i] = whole.dst + at;
            batch.len[i] = static_cast<int32_t>(len);
            batch.first_block[i + 1] = batch.first_block[i] + static_cast<int32_t>(chunks);
            batch.n = i + 1;
            if (batch.n == kSegs) {
                const zero_status st = flush();
                if (st != ZERO_OK) return st;
            }
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

// One launch per Batch::kTens tensors of a Shard(0) plan. bufs: the N_d rank
// buffers; tensors: the T tensors. kScatter picks the direction.
template <bool kScatter, class Batch>
zero_status launch_tensors(const zero_plan* plan, uint16_t* const* bufs, uint16_t* const* tensors,
                           hipStream_t stream, const char* who) {
    Batch batch{};
    for (int32_t r = 0; r < plan->n_ranks; ++r) batch.shards[r] = bufs[r];
    auto flush = [&]() -> zero_status {
        if (batch.n == 0) return ZERO_OK;
        const int64_t blocks = batch.first_block[batch.n];
        hipLaunchKernelGGL((gather_tensor_kernel<kScatter, Batch>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kThreads), 0, stream, batch);
        batch.n = 0;
        batch.first_block[0] = 0;
        return zero::check_hip(hipGetLastError(), who);
    };
    for (size_t t = 0; t < plan->numels.size(); ++t) {
        const int64_t n = plan->numels[t];
        if (n <= 0) continue;
        const int64_t blocks = (n + kChunk - 1) / kChunk;
        if (int64_t(batch.first_block[batch.n]) + blocks > 0x7FFFFFFF) {
            const zero_status st = flush();
            if (st != ZERO_OK) return st;
        }
        const int i = batch.n;
        batch.dst[i] = tensors[t];
        batch.numel[i] = static_cast<int32_t>(n);
        batch.chunk[i] = static_cast<int32_t>(plan->chunk_elems[t]);
        batch.off[i] = static_cast<typename Batch::OffT>(plan->offsets[t]);
        batch.first_block[i + 1] = batch.first_block[i] + static_cast<int32_t>(blocks);
        batch.n = i + 1;
        if (batch.n == Batch::kTens) {
            const zero_status st = flush();
            if (st != ZERO_OK) return st;
        }
    }
    return flush();
}

using zero::copy::flatten_pieces;
using zero::copy::gather_pieces;

using zero::copy::fits_compact;
using zero::copy::fits_tensor_major;

template <bool kScatter>
zero_status launch_tensors_any(const zero_plan* plan, uint16_t* const* bufs,
                               uint16_t* const* tensors, hipStream_t stream, const char* who) {
    return fits_compact(plan)
               ? launch_tensors<kScatter, CompactBatch>(plan, bufs, tensors, stream, who)
               : launch_tensors<kScatter, WideBatch>(plan, bufs, tensors, stream, who);
}

}  // namespace

// Shard(0) plans use the tensor-major kernel (ZERO_GATHER_TENSOR_MAJOR=0
// forces segment copies); flat plans copy segments (measured faster there).
#ifndef ZERO_GATHER_TENSOR_MAJOR
#define ZERO_GATHER_TENSOR_MAJOR 1
#endif

extern "C" zero_status zero_gather_params(const zero_plan* plan, const uint16_t* const* shards,
                                          uint16_t* const* tensors, hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (plan == nullptr || shards == nullptr)
        return fail(ZERO_EINVAL, "zero_gather_params: NULL plan or shards");
    zero_status st = check_tensors(plan, tensors, "zero_gather_params");
    if (st != ZERO_OK) return st;
    try {
        st = zero::copy::check_gather_ranges(plan, shards, tensors, "zero_gather_params");
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_gather_params: allocation failed");
    }
    if (st != ZERO_OK) return st;
    // A NULL shard skips that rank's segments (a caller gathers ranks as their
    // shards become ready, or the others while the own shard is still updated).
    bool all_present = true;
    for (int32_t r = 0; r < plan->n_ranks; ++r) all_present = all_present && shards[r] != nullptr;
    if (all_present && ZERO_GATHER_TENSOR_MAJOR && fits_tensor_major(plan))
        return launch_tensors_any<false>(plan, const_cast<uint16_t* const*>(shards), tensors, stream,
                                         "zero_gather_params launch");
    std::vector<Piece> pieces;
    try {
        pieces = gather_pieces(plan, shards, tensors);
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_gather_params: allocation failed");
    }
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
    try {
        st = zero::copy::check_flatten_ranges(plan, tensors, flat, "zero_flatten_params");
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_flatten_params: allocation failed");
    }
    if (st != ZERO_OK) return st;
    // Every gap between segments (and after the last) is filled with zeros;
    // Shard(0) plans copy the tensors with the tensor-major kernel, flat plans
    // copy every segment, in flat order, to its place.
    const bool tensor_major = ZERO_GATHER_TENSOR_MAJOR && fits_tensor_major(plan);
    std::vector<Piece> pieces;
    try {
        pieces = flatten_pieces(plan, tensors, flat, !tensor_major);
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_flatten_params: allocation failed");
    }
    if (tensor_major) {
        st = launch_pieces(pieces, stream, "zero_flatten_params launch");   // the gaps
        if (st != ZERO_OK) return st;
        std::vector<uint16_t*> bufs(static_cast<size_t>(plan->n_ranks));
        for (int32_t r = 0; r < plan->n_ranks; ++r) bufs[static_cast<size_t>(r)] = flat + int64_t(r) * plan->shard;
        return launch_tensors_any<true>(plan, bufs.data(), const_cast<uint16_t* const*>(tensors),
                                        stream, "zero_flatten_params launch");
    }
    return launch_pieces(pieces, stream, "zero_flatten_params launch");
}

// ------------------------------------------------------------ device table

struct zero_copy_table {
    int device = -1;
    void* mem = nullptr;          // descriptors, then the per-workgroup index
    const PieceDesc* table = nullptr;
    const uint32_t* index = nullptr;
    int64_t blocks = 0;
};

namespace {

zero_status make_copy_table(const std::vector<Piece>& pieces, zero_copy_table** out, const char* who) {
    using zero::fail;
    std::vector<PieceDesc> descs;
    std::vector<uint32_t> index;
    zero_copy_table* tab = nullptr;
    try {
        int64_t blocks = 0;
        // Piece order in the table, so in dispatch order: 0 (default) the plan's flat
        // order (the source shards front to back); 1 by destination address.
#ifndef ZERO_TABLE_BY_DESTINATION
#define ZERO_TABLE_BY_DESTINATION 0
#endif
        std::vector<Piece> ordered;
        if (ZERO_TABLE_BY_DESTINATION) {
            ordered = pieces;
            std::stable_sort(ordered.begin(), ordered.end(),
                             [](const Piece& a, const Piece& b) { return a.dst < b.dst; });
        }
        const zero_status cs = zero::copy::copy_table_contents(
            ZERO_TABLE_BY_DESTINATION ? ordered : pieces, kChunk, &descs, &index, &blocks, who);
        if (cs != ZERO_OK) return cs;
        tab = new zero_copy_table;
        tab->blocks = blocks;
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, std::string(who) + ": host allocation failed");
    }
    zero_status st = ZERO_OK;
    if (tab->blocks > 0) {        // an empty table needs no device
        st = zero::check_hip(hipGetDevice(&tab->device), who);
        const size_t table_bytes = (descs.size() * sizeof(PieceDesc) + 255) / 256 * 256;
        if (st == ZERO_OK)
            st = zero::check_hip(hipMalloc(&tab->mem, table_bytes + index.size() * sizeof(uint32_t)), who);
        if (st == ZERO_OK) {
            tab->table = static_cast<const PieceDesc*>(tab->mem);
            tab->index = reinterpret_cast<const uint32_t*>(static_cast<char*>(tab->mem) + table_bytes);
            st = zero::check_hip(hipMemcpy(tab->mem, descs.data(), descs.size() * sizeof(PieceDesc),
                                           hipMemcpyHostToDevice), who);
        }
        if (st == ZERO_OK)
            st = zero::check_hip(hipMemcpy(const_cast<uint32_t*>(tab->index), index.data(),
                                           index.size() * sizeof(uint32_t), hipMemcpyHostToDevice), who);
    }
    if (st != ZERO_OK) {
        if (tab->mem) (void)hipFree(tab->mem);
        delete tab;
        return st;
    }
    *out = tab;
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_gather_table_create(const zero_plan* plan, const uint16_t* const* shards,
                                                uint16_t* const* tensors, zero_copy_table** out) {
    using zero::fail;
    zero::clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "zero_gather_table_create: NULL out");
    *out = nullptr;
    if (plan == nullptr || shards == nullptr)
        return fail(ZERO_EINVAL, "zero_gather_table_create: NULL plan or shards");
    zero_status st = check_tensors(plan, tensors, "zero_gather_table_create");
    if (st != ZERO_OK) return st;
    std::vector<Piece> pieces;
    try {
        st = zero::copy::check_gather_ranges(plan, shards, tensors, "zero_gather_table_create");
        if (st != ZERO_OK) return st;
        pieces = gather_pieces(plan, shards, tensors);
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_gather_table_create: allocation failed");
    }
    return make_copy_table(pieces, out, "zero_gather_table_create");
}

extern "C" zero_status zero_flatten_table_create(const zero_plan* plan, const uint16_t* const* tensors,
                                                 uint16_t* flat, zero_copy_table** out) {
    using zero::fail;
    zero::clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "zero_flatten_table_create: NULL out");
    *out = nullptr;
    if (plan == nullptr) return fail(ZERO_EINVAL, "zero_flatten_table_create: NULL plan");
    if (plan->padded > 0 && flat == nullptr)
        return fail(ZERO_EINVAL, "zero_flatten_table_create: NULL flat");
    zero_status st = check_tensors(plan, tensors, "zero_flatten_table_create");
    if (st != ZERO_OK) return st;
    std::vector<Piece> pieces;
    try {
        st = zero::copy::check_flatten_ranges(plan, tensors, flat, "zero_flatten_table_create");
        if (st != ZERO_OK) return st;
        pieces = flatten_pieces(plan, tensors, flat, true);
    } catch (const std::bad_alloc&) {
        return fail(ZERO_ENOMEM, "zero_flatten_table_create: allocation failed");
    }
    return make_copy_table(pieces, out, "zero_flatten_table_create");
}

extern "C" zero_status zero_copy_table_run(const zero_copy_table* table, hipStream_t stream) {
    using zero::fail;
    zero::clear_error();
    if (table == nullptr) return fail(ZERO_EINVAL, "zero_copy_table_run: NULL table");
    if (table->blocks == 0) return ZERO_OK;
    int dev = -1;
    zero_status st = zero::check_hip(hipGetDevice(&dev), "zero_copy_table_run: hipGetDevice");
    if (st != ZERO_OK) return st;
    if (dev != table->device)
        return fail(ZERO_EINVAL, "zero_copy_table_run: the table lives on device " +
                                     std::to_string(table->device) + ", the current device is " +
                                     std::to_string(dev));
    // A dispatch holds fewer than 2^32 work-items: longer tables take several launches.
    constexpr int64_t kMaxBlocks = zero::kTableLaunchBlocks;
    for (int64_t b0 = 0; b0 < table->blocks; b0 += kMaxBlocks) {
        const int64_t nb = table->blocks - b0 < kMaxBlocks ? table->blocks - b0 : kMaxBlocks;
        const int64_t per = (nb + 7) / 8;
        hipLaunchKernelGGL(copy_table_kernel, dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0,
                           stream, table->table, table->index, b0, per);
        st = zero::check_hip(hipGetLastError(), "zero_copy_table_run launch");
        if (st != ZERO_OK) return st;
    }
    return ZERO_OK;
}

extern "C" int64_t zero_copy_table_blocks(const zero_copy_table* table) {
    return table ? table->blocks : -1;
}

extern "C" void zero_copy_table_free(zero_copy_table* table) {
    if (!table) return;
    if (table->mem) (void)hipFree(table->mem);
    delete table;
}
