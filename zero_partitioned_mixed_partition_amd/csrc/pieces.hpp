// Host-side piece lists of the bf16 gather and flatten copies, and the
// contents of a device copy table and of a reduce table (host C++, no device
// code).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "Execution Flow for ZeRO-1", step 4
// (the gather) and section "FSDP-1: FlatParameter and Module-Level Wrapping"
// (the flatten): every plan segment is one piece, copied between its place in
// a rank's shard and its place in its tensor; the flatten also zero-fills every
// gap of the flat buffer.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "internal.hpp"

namespace zero {
namespace copy {

// len elements from src to dst; a NULL src fills dst with zeros.
struct Piece {
    const uint16_t* src;
    uint16_t* dst;
    int64_t len;
};

// A copy table's descriptor of one piece: the piece and its first workgroup.
struct alignas(32) PieceDesc {
    const uint16_t* src;        // NULL: fill with zeros
    uint16_t* dst;
    int64_t len;
    int64_t first_block;
};
static_assert(sizeof(PieceDesc) == 32, "one 32-byte descriptor per piece");

// Every segment of the plan as a piece from its shard to its tensor (a NULL
// shard skips its rank's segments). Throws std::bad_alloc.
std::vector<Piece> gather_pieces(const zero_plan* plan, const uint16_t* const* shards,
                                 uint16_t* const* tensors);

// Every segment from its tensor to its place in the flat buffer, in flat order,
// with a zero-fill piece for every gap (and after the last segment). With
// with_copies false, the gaps only. Throws std::bad_alloc.
std::vector<Piece> flatten_pieces(const zero_plan* plan, const uint16_t* const* tensors,
                                  uint16_t* flat, bool with_copies);

// A copy table's contents for `pieces`, at `chunk` elements per workgroup: one
// descriptor per non-empty piece, and the XCD-major per-workgroup descriptor
// index (xcd_major_index). ZERO_ERANGE past 2^31 workgroups; throws
// std::bad_alloc.
zero_status copy_table_contents(const std::vector<Piece>& pieces, int64_t chunk,
                                std::vector<PieceDesc>* descs, std::vector<uint32_t>* index,
                                int64_t* blocks, const char* who);

// A reduce table's descriptor of one piece of the rank's shard: a segment
// (elements [src_off, src_off + len) of tensor `tensor` in every replica, into
// shard elements [dst_off, dst_off + len)) or a gap of padding (tensor -1,
// written as zeros), with its first workgroup and whether 16-byte accesses
// apply (every replica's tensor 16-byte aligned, both offsets multiples of 8,
// the shard 16-byte aligned).
struct alignas(64) RPieceDesc {
    int64_t src_off;
    int64_t dst_off;
    int64_t len;
    int64_t first_block;
    int32_t tensor;
    int32_t vec;
    int64_t unused[2];
};
static_assert(sizeof(RPieceDesc) == 64, "one 64-byte descriptor per piece");

// A reduce table's contents for `rank` of `plan`, at `chunk` shard elements
// per workgroup: the rank's segments and the padding gaps around them, in
// shard order, as descriptors; the XCD-major per-workgroup descriptor index
// (xcd_major_index); and the R * T replica pointers tensor-major (pointer of
// replica k's tensor t at t * R + k; replica_tensors holds it at k * T + t).
// ZERO_EINVAL for a NULL replica tensor that a segment needs, or one that
// overlaps shard_grad's S elements; ZERO_ERANGE past 2^31 workgroups; throws
// std::bad_alloc.
zero_status reduce_table_contents(const zero_plan* plan, int32_t rank,
                                  const uint16_t* const* replica_tensors, int32_t n_replicas,
                                  const uint16_t* shard_grad, int64_t chunk,
                                  std::vector<RPieceDesc>* descs, std::vector<uint32_t>* index,
                                  std::vector<const uint16_t*>* ptrs, int64_t* blocks_out,
                                  const char* who);

// first_overlap for long lists (a gather's tensors and shards): "<a> overlaps
// <b>" for a written range that shares bytes with another written range or
// with a read range, or an empty string. Ranges with a NULL pointer or no
// bytes are left out. Sorts the written ranges, so O((W + R) log W). Throws
// std::bad_alloc.
std::string first_overlap_sorted(std::vector<Span> written, const std::vector<Span>& read);

// The gather's ranges: tensor t (numel_t elements) is written, each non-NULL
// shard (S elements) is read. ZERO_EINVAL naming the first overlap; throws
// std::bad_alloc.
zero_status check_gather_ranges(const zero_plan* plan, const uint16_t* const* shards,
                                uint16_t* const* tensors, const char* who);

// The flatten's ranges: the flat buffer (P elements) is written, each tensor
// read. ZERO_EINVAL naming the first overlap; throws std::bad_alloc.
zero_status check_flatten_ranges(const zero_plan* plan, const uint16_t* const* tensors,
                                 const uint16_t* flat, const char* who);

}  // namespace copy
}  // namespace zero
