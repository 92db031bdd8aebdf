// Host-side piece lists and copy-table contents (see pieces.hpp).
#include "pieces.hpp"

#include <algorithm>
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

zero_status reduce_table_contents(const zero_plan* plan, int32_t rank,
                                  const uint16_t* const* replica_tensors, int32_t n_replicas,
                                  const uint16_t* shard_grad, int64_t chunk,
                                  std::vector<RPieceDesc>* descs, std::vector<uint32_t>* index,
                                  std::vector<const uint16_t*>* ptrs, int64_t* blocks_out,
                                  const char* who) {
    descs->clear();
    index->clear();
    const int64_t T = static_cast<int64_t>(plan->numels.size());
    const std::vector<zero_segment>& segs = plan->by_rank[static_cast<size_t>(rank)];
    ptrs->assign(static_cast<size_t>(T * n_replicas), nullptr);
    std::vector<char> vec_ok(static_cast<size_t>(T), 1);
    for (int64_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < n_replicas; ++k) {
            const uint16_t* q = replica_tensors[static_cast<int64_t>(k) * T + t];
            (*ptrs)[static_cast<size_t>(t * n_replicas + k)] = q;
            if ((reinterpret_cast<uintptr_t>(q) & 15) != 0) vec_ok[static_cast<size_t>(t)] = 0;
        }
    const bool out_ok = (reinterpret_cast<uintptr_t>(shard_grad) & 15) == 0;
    int64_t blocks = 0;
    auto add = [&](int32_t t, int64_t src_off, int64_t dst_off, int64_t len) -> zero_status {
        if (len <= 0) return ZERO_OK;
        const int64_t b = len / chunk + (len % chunk != 0 ? 1 : 0);
        if (b > 0x7FFFFFFF - blocks || descs->size() >= 0xFFFFFFFFu)
            return fail(ZERO_ERANGE, std::string(who) + ": more than 2^31 workgroups");
        RPieceDesc d{};
        d.src_off = src_off;
        d.dst_off = dst_off;
        d.len = len;
        d.first_block = blocks;
        d.tensor = t;
        d.vec = t >= 0 && out_ok && vec_ok[static_cast<size_t>(t)] && src_off % 8 == 0 && dst_off % 8 == 0;
        index->insert(index->end(), static_cast<size_t>(b), static_cast<uint32_t>(descs->size()));
        descs->push_back(d);
        blocks += b;
        return ZERO_OK;
    };
    const size_t out_bytes = static_cast<size_t>(plan->shard) * 2;
    int64_t pos = 0;
    for (const zero_segment& seg : segs) {
        if (seg.length <= 0) continue;
        for (int32_t k = 0; k < n_replicas; ++k) {
            const uint16_t* q = (*ptrs)[static_cast<size_t>(seg.tensor * static_cast<int64_t>(n_replicas) + k)];
            if (q == nullptr)
                return fail(ZERO_EINVAL, std::string(who) + ": NULL tensor " + std::to_string(seg.tensor) +
                                             " of replica " + std::to_string(k));
            const size_t q_bytes = static_cast<size_t>(plan->numels[static_cast<size_t>(seg.tensor)]) * 2;
            if (ranges_overlap(shard_grad, out_bytes, q, q_bytes))
                return fail(ZERO_EINVAL, std::string(who) + ": shard_grad overlaps tensor " +
                                             std::to_string(seg.tensor) + " of replica " + std::to_string(k));
        }
        zero_status st = add(-1, 0, pos, seg.shard_offset - pos);
        if (st == ZERO_OK) st = add(seg.tensor, seg.tensor_offset, seg.shard_offset, seg.length);
        if (st != ZERO_OK) return st;
        pos = seg.shard_offset + seg.length;
    }
    const zero_status st = add(-1, 0, pos, plan->shard - pos);
    if (st != ZERO_OK) return st;
    if (blocks > 0) *index = xcd_major_index(*index);
    *blocks_out = blocks;
    return ZERO_OK;
}

std::string first_overlap_sorted(std::vector<Span> written, const std::vector<Span>& read) {
    auto lo = [](const Span& x) { return reinterpret_cast<uintptr_t>(x.p); };
    written.erase(std::remove_if(written.begin(), written.end(),
                                 [](const Span& x) { return x.p == nullptr || x.bytes == 0; }),
                  written.end());
    std::sort(written.begin(), written.end(), [&](const Span& a, const Span& b) { return lo(a) < lo(b); });
    // Sorted by start, two ranges overlap only if some neighbours do.
    for (size_t i = 1; i < written.size(); ++i)
        if (lo(written[i]) < lo(written[i - 1]) + written[i - 1].bytes)
            return span_name(written[i - 1]) + " overlaps " + span_name(written[i]);
    // Now disjoint, so their ends rise with their starts: the one written range
    // that can meet [a, b) first is the first ending after a.
    for (const Span& r : read) {
        if (r.p == nullptr || r.bytes == 0) continue;
        const auto it = std::upper_bound(written.begin(), written.end(), lo(r),
                                         [&](uintptr_t a, const Span& w) { return a < lo(w) + w.bytes; });
        if (it != written.end() && lo(*it) < lo(r) + r.bytes) return span_name(*it) + " overlaps " + span_name(r);
    }
    return std::string();
}

zero_status check_gather_ranges(const zero_plan* plan, const uint16_t* const* shards,
                                uint16_t* const* tensors, const char* who) {
    std::vector<Span> wr, rd;
    wr.reserve(plan->numels.size());
    for (size_t t = 0; t < plan->numels.size(); ++t)
        wr.push_back({tensors[t], static_cast<size_t>(plan->numels[t]) * 2, "tensor", static_cast<int>(t)});
    for (int32_t r = 0; r < plan->n_ranks; ++r)
        rd.push_back({shards[r], static_cast<size_t>(plan->shard) * 2, "shard", r});
    const std::string clash = first_overlap_sorted(std::move(wr), rd);
    return clash.empty() ? ZERO_OK : fail(ZERO_EINVAL, std::string(who) + ": " + clash);
}

zero_status check_flatten_ranges(const zero_plan* plan, const uint16_t* const* tensors,
                                 const uint16_t* flat, const char* who) {
    std::vector<Span> rd;
    rd.reserve(plan->numels.size());
    for (size_t t = 0; t < plan->numels.size(); ++t)
        rd.push_back({tensors[t], static_cast<size_t>(plan->numels[t]) * 2, "tensor", static_cast<int>(t)});
    const std::string clash =
        first_overlap_sorted({{flat, static_cast<size_t>(plan->padded) * 2, "flat"}}, rd);
    return clash.empty() ? ZERO_OK : fail(ZERO_EINVAL, std::string(who) + ": " + clash);
}

}  // namespace copy
}  // namespace zero
