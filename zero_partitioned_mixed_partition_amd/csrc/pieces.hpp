// Host-side piece lists of the bf16 gather and flatten copies, and the
// contents of a device copy table (host C++, no device code).
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "Execution Flow for ZeRO-1", step 4
// (the gather) and section "FSDP-1: FlatParameter and Module-Level Wrapping"
// (the flatten): every plan segment is one piece, copied between its place in
// a rank's shard and its place in its tensor; the flatten also zero-fills every
// gap of the flat buffer.
#pragma once

#include <cstdint>
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

}  // namespace copy
}  // namespace zero
