// Internal declarations shared by the library's translation units.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "zero_mi355x.h"

struct zero_plan {
    int32_t kind = 0;     // ZERO_PLAN_FLAT or ZERO_PLAN_SHARD0
    int32_t n_ranks = 0;
    int32_t align = 0;
    int64_t numel = 0;    // Phi
    int64_t padded = 0;   // P (flat: padded flat length; Shard(0): N_d * S)
    int64_t shard = 0;    // S
    std::vector<int64_t> numels;
    std::vector<int64_t> offsets;   // flat: tensor start; Shard(0): chunk start within a shard
    std::vector<int64_t> chunk_elems;   // Shard(0): elements per full rank chunk (rows * row length)
    std::vector<std::vector<zero_segment>> by_rank;   // segments of each rank, flat order
    std::vector<zero_segment> all;                    // every segment, flat order
};

namespace zero {

// Records a readable detail for zero_last_error() and returns `st`.
zero_status fail(zero_status st, const std::string& detail);
// Maps a HIP error to ZERO_EHIP with its string, or returns ZERO_OK.
zero_status check_hip(int hip_error, const char* what);
// Clears the thread's last error (called on entry of each ABI function).
void clear_error();

// Compute units of the current device (cached per device).
int device_cu_count();

// Host-side argument checks: whether [a, a + a_bytes) and [b, b + b_bytes)
// share a byte.
inline bool ranges_overlap(const void* a, size_t a_bytes, const void* b, size_t b_bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return a_bytes > 0 && b_bytes > 0 && x < y + b_bytes && y < x + a_bytes;
}

// A device range an entry point reads or writes, named for the error message
// ("replica 3" when index >= 0).
struct Span {
    const void* p;
    size_t bytes;
    const char* name;
    int index = -1;
};

inline std::string span_name(const Span& s) {
    return s.index < 0 ? std::string(s.name) : std::string(s.name) + " " + std::to_string(s.index);
}

// The kernels read and write element i of every array from one lane, so a
// written range that shares bytes with another written range, or with a range
// they read, races. Returns "<a> overlaps <b>" for the first such pair, or an
// empty string; ranges that are only read may overlap one another.
inline std::string first_overlap(const Span* written, int n_written, const Span* read, int n_read) {
    for (int i = 0; i < n_written; ++i) {
        for (int j = i + 1; j < n_written; ++j)
            if (ranges_overlap(written[i].p, written[i].bytes, written[j].p, written[j].bytes))
                return span_name(written[i]) + " overlaps " + span_name(written[j]);
        for (int j = 0; j < n_read; ++j)
            if (ranges_overlap(written[i].p, written[i].bytes, read[j].p, read[j].bytes))
                return span_name(written[i]) + " overlaps " + span_name(read[j]);
    }
    return std::string();
}

// Device-resident tables (multi-tensor AdamW, gather/flatten copies) hold one
// descriptor index per workgroup. The dispatcher deals a launch's workgroups
// round-robin to the 8 XCDs, so the index is stored XCD-major within each
// launch: workgroup x of a launch of nb reads entry (x % 8) * per + x / 8,
// per = ceil(nb / 8). Each XCD then reads one contiguous run and each index
// line is fetched once, instead of once per XCD. Launches hold a multiple of 8
// workgroups (all but the last), so launch j's entries start at its first
// workgroup; the last launch pads its run by at most 7 entries.
constexpr int64_t kTableLaunchBlocks = ((int64_t(1) << 32) / 256 - 1) / 8 * 8;

// The XCD-major index of `plain` (entry b = descriptor of workgroup b).
inline std::vector<uint32_t> xcd_major_index(const std::vector<uint32_t>& plain) {
    const int64_t total = static_cast<int64_t>(plain.size());
    std::vector<uint32_t> out(plain.size() + 7, 0u);
    for (int64_t b0 = 0; b0 < total; b0 += kTableLaunchBlocks) {
        const int64_t nb = total - b0 < kTableLaunchBlocks ? total - b0 : kTableLaunchBlocks;
        const int64_t per = (nb + 7) / 8;
        for (int64_t x = 0; x < nb; ++x)
            out[static_cast<size_t>(b0 + (x % 8) * per + x / 8)] = plain[static_cast<size_t>(b0 + x)];
    }
    return out;
}

}  // namespace zero
