// Host-side piece lists and copy-table contents (see pieces.hpp).
#include "pieces.hpp"

#include <string>

namespace zero {
namespace copy {

std::vector<Piece> gather_pieces(const zero_plan* plan, const uint16_t* const* shards,
                                 uint16_t* const* tensors) {
    std::vector<Piece> pieces;
    pieces.reserve(plan->all.size());
    for (const zero_segment& seg : plan->all)
        if (shards[seg.rank] != nullptr)
            pieces.push_back({shards[seg.rank] + seg.shard_offset,
                              tensors[seg.tensor] + seg.tensor_offset, seg.length});
    return pieces;
}

std::vector<Piece> flatten_pieces(const zero_plan* plan, const uint16_t* const* tensors,
                                  uint16_t* flat, bool with_copies) {
    std::vector<Piece> pieces;
    pieces.reserve(2 * plan->all.size() + 1);
    int64_t pos = 0;
    for (const zero_segment& seg : plan->all) {
        const int64_t at = static_cast<int64_t>(seg.rank) * plan->shard + seg.shard_offset;
        if (at > pos) pieces.push_back({nullptr, flat + pos, at - pos});
        if (with_copies)
            pieces.push_back({tensors[seg.tensor] + seg.tensor_offset, flat + at, seg.length});
        pos = at + seg.length;
    }
    if (plan->padded > pos) pieces.push_back({nullptr, flat + pos, plan->padded - pos});
    return pieces;
}

zero_status copy_table_contents(const std::vector<Piece>& pieces, int64_t chunk,
                                std::vector<PieceDesc>* descs, std::vector<uint32_t>* index,
                                int64_t* blocks_out, const char* who) {
    descs->clear();
    index->clear();
    int64_t blocks = 0;
    for (const Piece& pc : pieces) {
        if (pc.len <= 0) continue;
        const int64_t b = pc.len / chunk + (pc.len % chunk != 0 ? 1 : 0);
        if (b > 0x7FFFFFFF - blocks || descs->size() >= 0xFFFFFFFFu)
            return fail(ZERO_ERANGE, std::string(who) + ": more than 2^31 workgroups");
        index->insert(index->end(), static_cast<size_t>(b), static_cast<uint32_t>(descs->size()));
        descs->push_back({pc.src, pc.dst, pc.len, blocks});
        blocks += b;
    }
    if (blocks > 0) *index = xcd_major_index(*index);
    *blocks_out = blocks;
    return ZERO_OK;
}

}  // namespace copy
}  // namespace zero
