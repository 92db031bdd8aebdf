// Partition plans (host only): the flat FSDP-1 / ZeRO layout, and FSDP-2's
// per-parameter Shard(0) layout further below.
//
// "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data Parallelism (FSDP):
// Mathematical Foundations ...", section "FSDP-1: FlatParameter and
// Module-Level Wrapping": tensors are flattened in order into one 1-D buffer,
// padded at the end to a length divisible by N_d, and cut into N_d equal
// chunks. The padded length is also a multiple of N_d*A, so each shard holds a
// whole number of A-element units and every shard starts on an A boundary.
//
// Segments are produced by one merge over the tensor and shard boundaries:
// O(T + N_d) time and space.
#include <cmath>
#include <new>
#include <string>

#include "internal.hpp"

using zero::clear_error;
using zero::fail;

extern "C" zero_status zero_partition_plan(const int64_t* numels, int32_t n_tensors,
                                           int32_t n_ranks, int32_t align_elems,
                                           zero_plan** out) {
    clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "zero_partition_plan: out is NULL");
    *out = nullptr;
    if (n_tensors < 0) return fail(ZERO_EINVAL, "zero_partition_plan: n_tensors < 0");
    if (n_tensors > 0 && numels == nullptr)
        return fail(ZERO_EINVAL, "zero_partition_plan: numels is NULL");
    if (n_ranks < 1) return fail(ZERO_EINVAL, "zero_partition_plan: n_ranks < 1");
    if (align_elems < 1) return fail(ZERO_EINVAL, "zero_partition_plan: align_elems < 1");

    zero_plan* plan = new (std::nothrow) zero_plan;
    if (plan == nullptr) return fail(ZERO_ENOMEM, "zero_partition_plan: allocation failed");
    try {
        plan->n_ranks = n_ranks;
        plan->align = align_elems;
        plan->numels.assign(numels, numels + n_tensors);
        plan->offsets.resize(static_cast<size_t>(n_tensors));
        int64_t total = 0;
        for (int32_t t = 0; t < n_tensors; ++t) {
            const int64_t n = numels[t];
            if (n < 0) {
                delete plan;
                return fail(ZERO_EINVAL, "zero_partition_plan: numels[" + std::to_string(t) +
                                             "] < 0");
            }
            if (n > INT64_MAX - total) {
                delete plan;
                return fail(ZERO_ERANGE, "zero_partition_plan: total numel overflows int64");
            }
            plan->offsets[static_cast<size_t>(t)] = total;
            total += n;
        }
        const int64_t unit = static_cast<int64_t>(n_ranks) * align_elems;
        const int64_t units = total / unit + (total % unit != 0 ? 1 : 0);
        if (units > INT64_MAX / unit) {
            delete plan;
            return fail(ZERO_ERANGE, "zero_partition_plan: padded length overflows int64");
        }
        plan->numel = total;
        plan->padded = units * unit;
        plan->shard = plan->padded / n_ranks;

        plan->by_rank.assign(static_cast<size_t>(n_ranks), {});
        const int64_t s = plan->shard;
        // Walk the tensors in flat order; split each at the shard boundaries it spans.
        for (int32_t t = 0; t < n_tensors; ++t) {
            int64_t lo = plan->offsets[static_cast<size_t>(t)];
            const int64_t hi = lo + plan->numels[static_cast<size_t>(t)];
            while (lo < hi) {
                const int64_t r = lo / s;
                const int64_t shard_end = (r + 1) * s;
                const int64_t end = hi < shard_end ? hi : shard_end;
                zero_segment seg;
                seg.tensor = t;
                seg.rank = static_cast<int32_t>(r);
                seg.tensor_offset = lo - plan->offsets[static_cast<size_t>(t)];
                seg.shard_offset = lo - r * s;
                seg.length = end - lo;
                plan->by_rank[static_cast<size_t>(r)].push_back(seg);
                plan->all.push_back(seg);
                lo = end;
            }
        }
    } catch (const std::bad_alloc&) {
        delete plan;
        return fail(ZERO_ENOMEM, "zero_partition_plan: allocation failed");
    }
    *out = plan;
    return ZERO_OK;
}

// FSDP-2 Shard(0): "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data
// Parallelism (FSDP): Mathematical Foundations ...", section "FSDP-2:
// Per-Parameter Sharding via DTensor (fully_shard)": every tensor is sharded on
// its own along dim 0; one rank's shards share a coalesced buffer. Chunks of
// ceil(dim0 / N_d) rows, as torch.chunk cuts them; each padded to full size.
extern "C" zero_status zero_partition_plan_shard0(const int64_t* numels, const int64_t* dim0,
                                                  int32_t n_tensors, int32_t n_ranks,
                                                  int32_t align_elems, zero_plan** out) {
    clear_error();
    if (out == nullptr) return fail(ZERO_EINVAL, "zero_partition_plan_shard0: out is NULL");
    *out = nullptr;
    if (n_tensors < 0) return fail(ZERO_EINVAL, "zero_partition_plan_shard0: n_tensors < 0");
    if (n_tensors > 0 && (numels == nullptr || dim0 == nullptr))
        return fail(ZERO_EINVAL, "zero_partition_plan_shard0: numels or dim0 is NULL");
    if (n_ranks < 1) return fail(ZERO_EINVAL, "zero_partition_plan_shard0: n_ranks < 1");
    if (align_elems < 1) return fail(ZERO_EINVAL, "zero_partition_plan_shard0: align_elems < 1");
    zero_plan* plan = new (std::nothrow) zero_plan;
    if (plan == nullptr) return fail(ZERO_ENOMEM, "zero_partition_plan_shard0: allocation failed");
    try {
        plan->kind = 1;
        plan->n_ranks = n_ranks;
        plan->align = align_elems;
        plan->numels.assign(numels, numels + n_tensors);
        plan->offsets.resize(static_cast<size_t>(n_tensors));
        std::vector<int64_t> chunk_rows(static_cast<size_t>(n_tensors)), inner(chunk_rows.size());
        int64_t total = 0, buf = 0;
        for (int32_t t = 0; t < n_tensors; ++t) {
            const int64_t n = numels[t], d0 = dim0[t];
            if (n < 0 || d0 < 0 || (n > 0 && (d0 == 0 || n % d0 != 0))) {
                delete plan;
                return fail(ZERO_EINVAL, "zero_partition_plan_shard0: tensor " + std::to_string(t) +
                                             ": dim0 must be >= 1 and divide numel");
            }
            const int64_t in = n > 0 ? n / d0 : 0;
            const int64_t rows = n > 0 ? d0 / n_ranks + (d0 % n_ranks != 0 ? 1 : 0) : 0;
            if (n > INT64_MAX - total || (in > 0 && rows > (INT64_MAX - buf) / in)) {
                delete plan;
                return fail(ZERO_ERANGE, "zero_partition_plan_shard0: sizes overflow int64");
            }
            total += n;
            chunk_rows[static_cast<size_t>(t)] = rows;
            inner[static_cast<size_t>(t)] = in;
            plan->offsets[static_cast<size_t>(t)] = buf;
            plan->chunk_elems.push_back(rows * in);
            buf += rows * in;
        }
        if (buf > INT64_MAX - (align_elems - 1)) {
            delete plan;
            return fail(ZERO_ERANGE, "zero_partition_plan_shard0: padded length overflows int64");
        }
        const int64_t s = (buf + align_elems - 1) / align_elems * align_elems;
        if (s > INT64_MAX / n_ranks) {
            delete plan;
            return fail(ZERO_ERANGE, "zero_partition_plan_shard0: padded length overflows int64");
        }
        plan->numel = total;
        plan->shard = s;
        plan->padded = s * n_ranks;
        plan->by_rank.assign(static_cast<size_t>(n_ranks), {});
        for (int32_t r = 0; r < n_ranks; ++r) {
            for (int32_t t = 0; t < n_tensors; ++t) {
                const size_t ti = static_cast<size_t>(t);
                const int64_t d0 = plan->numels[ti] > 0 ? dim0[t] : 0;
                // rank r holds rows only if r * chunk_rows < d0 (checked without the product)
                if (d0 == 0 || r > (d0 - 1) / chunk_rows[ti]) continue;
                const int64_t first = static_cast<int64_t>(r) * chunk_rows[ti];
                const int64_t rows = d0 - first < chunk_rows[ti] ? d0 - first : chunk_rows[ti];
                if (rows <= 0) continue;
                zero_segment seg;
                seg.tensor = t;
                seg.rank = r;
                seg.tensor_offset = first * inner[ti];
                seg.shard_offset = plan->offsets[ti];
                seg.length = rows * inner[ti];
                plan->by_rank[static_cast<size_t>(r)].push_back(seg);
                plan->all.push_back(seg);
            }
        }
    } catch (const std::bad_alloc&) {
        delete plan;
        return fail(ZERO_ENOMEM, "zero_partition_plan_shard0: allocation failed");
    }
    *out = plan;
    return ZERO_OK;
}

extern "C" int32_t zero_plan_kind(const zero_plan* p) { return p ? p->kind : -1; }

extern "C" void zero_plan_free(zero_plan* plan) { delete plan; }

extern "C" int64_t zero_plan_numel(const zero_plan* p) { return p ? p->numel : -1; }
extern "C" int64_t zero_plan_padded_numel(const zero_plan* p) { return p ? p->padded : -1; }
extern "C" int64_t zero_plan_shard_numel(const zero_plan* p) { return p ? p->shard : -1; }
extern "C" int32_t zero_plan_num_tensors(const zero_plan* p) {
    return p ? static_cast<int32_t>(p->numels.size()) : -1;
}
extern "C" int32_t zero_plan_num_ranks(const zero_plan* p) { return p ? p->n_ranks : -1; }

extern "C" int64_t zero_plan_tensor_offset(const zero_plan* p, int32_t t) {
    if (p == nullptr || t < 0 || static_cast<size_t>(t) >= p->offsets.size()) return -1;
    return p->offsets[static_cast<size_t>(t)];
}

extern "C" int64_t zero_plan_tensor_numel(const zero_plan* p, int32_t t) {
    if (p == nullptr || t < 0 || static_cast<size_t>(t) >= p->numels.size()) return -1;
    return p->numels[static_cast<size_t>(t)];
}

extern "C" int32_t zero_plan_num_segments(const zero_plan* p, int32_t rank) {
    if (p == nullptr || rank < 0 || rank >= p->n_ranks) return -1;
    return static_cast<int32_t>(p->by_rank[static_cast<size_t>(rank)].size());
}

extern "C" zero_status zero_plan_segments(const zero_plan* p, int32_t rank, zero_segment* out,
                                          int32_t capacity, int32_t* count) {
    clear_error();
    if (p == nullptr || count == nullptr)
        return fail(ZERO_EINVAL, "zero_plan_segments: NULL plan or count");
    if (rank < 0 || rank >= p->n_ranks)
        return fail(ZERO_EINVAL, "zero_plan_segments: rank out of range");
    const auto& segs = p->by_rank[static_cast<size_t>(rank)];
    *count = static_cast<int32_t>(segs.size());
    if (static_cast<int64_t>(segs.size()) > capacity)
        return fail(ZERO_ENOSPACE, "zero_plan_segments: capacity too small");
    if (!segs.empty() && out == nullptr) return fail(ZERO_EINVAL, "zero_plan_segments: out is NULL");
    for (size_t i = 0; i < segs.size(); ++i) out[i] = segs[i];
    return ZERO_OK;
}

extern "C" zero_status zero_plan_memory_bytes(const zero_plan* p, int32_t stage, int32_t padded,
                                              double* bytes) {
    clear_error();
    if (p == nullptr || bytes == nullptr)
        return fail(ZERO_EINVAL, "zero_plan_memory_bytes: NULL argument");
    const double phi = static_cast<double>(p->numel);
    const double nd = static_cast<double>(p->n_ranks);
    const double pp = static_cast<double>(p->padded);
    const double s = static_cast<double>(p->shard);
    switch (stage) {
        case 0: *bytes = 16.0 * phi; break;
        case 1: *bytes = padded ? 4.0 * pp + 12.0 * s : 4.0 * phi + 12.0 * phi / nd; break;
        case 2: *bytes = padded ? 2.0 * pp + 14.0 * s : 2.0 * phi + 14.0 * phi / nd; break;
        case 3: *bytes = padded ? 16.0 * s : 16.0 * phi / nd; break;
        default: return fail(ZERO_EINVAL, "zero_plan_memory_bytes: stage must be 0..3");
    }
    return ZERO_OK;
}
