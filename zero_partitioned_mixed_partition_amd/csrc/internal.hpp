// Internal declarations shared by the library's translation units.
#pragma once

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
