// Host model of every streaming store the library's kernels make: for each
// kernel, the addresses one wave stores to, computed from the kernel's own
// indexing, checked against the contract of the store form the kernel uses
// (device_common.hpp):
//   st_stream(p, v)         base = first active lane's address - 2 GiB: every
//                           active lane's access must end within 2^32 - 1 bytes
//                           of that base and start at or above it;
//   st_stream_at(b, off, v) wave-uniform base b: every access must end within
//                           2^32 - 1 bytes of b;
//   st_stream_any(p, v)     global store: no constraint.
// The tensor-major copy (gather.hip) runs its real index map and routing
// (tensor_major.hpp) on plans built by the real planner (plan.cpp); its waves
// are enumerated wherever the rank can change inside a wave, and each element's
// place is also checked against the definition (rank e / chunk, offset
// e % chunk). The other kernels store one contiguous run per wave; their runs
// are modelled from their index formulas at the first and last wave of every
// launch.
//
// Input (stdin): lines "plan <kind> <n_ranks> <align> <n_tensors>" followed by
// n_tensors lines "<numel> <dim0>"; kind 0 = flat, 1 = Shard(0).
// Output: one line per plan with its route and the widest span seen per form,
// then "ok", or a line starting "FAIL".
#include <cinttypes>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.hpp"
#include "tensor_major.hpp"

namespace {

constexpr uint64_t kTwo31 = uint64_t(1) << 31;
constexpr uint64_t kMaxOff = 0xFFFFFFFFull;   // the buffer's record count

// Pointers the model hands the kernels: 256-byte aligned, as HIP allocations.
constexpr uint64_t kFlatBase = 0x7f0000000000ull;
constexpr uint64_t kTensorBase = 0x7e0000000000ull;
constexpr uint64_t kStateBase = 0x7c0000000000ull;

int g_fail = 0;

void fail(const std::string& what) {
    if (g_fail++ < 20) printf("FAIL %s\n", what.c_str());
}

// One wave's accesses through the first store form: (address, bytes) of its
// active lanes in lane order. Returns the span from the first active lane
// (the largest distance either way), for the report.
uint64_t check_first_lane_form(const std::vector<std::pair<uint64_t, uint64_t>>& acc,
                               const char* who) {
    if (acc.empty()) return 0;
    const uint64_t first = acc[0].first;
    const uint64_t base = first >= kTwo31 ? first - kTwo31 : 0;
    uint64_t span = 0;
    for (const auto& a : acc) {
        const uint64_t d = a.first > first ? a.first - first + a.second : first - a.first;
        if (d > span) span = d;
        if (a.first < base || a.first - base + a.second > kMaxOff) {
            fail(std::string(who) + ": a lane stores outside its wave's 32-bit window");
            return span;
        }
    }
    return span;
}

struct Report {
    uint64_t first_lane_span = 0;   // widest st_stream wave
    uint64_t at_max_end = 0;        // largest st_stream_at offset + bytes
    uint64_t old_form_span = 0;     // the flatten's waves as st_stream would have seen them
    int64_t waves = 0;
    int64_t elems_checked = 0;
};

// A contiguous run of `lanes` accesses of `bytes` each, `stride` bytes apart,
// from `addr` (AdamW, the reduce, the piece copies, the gather into a tensor).
void check_run(uint64_t addr, int lanes, uint64_t stride, uint64_t bytes, const char* who,
               Report& rep) {
    std::vector<std::pair<uint64_t, uint64_t>> acc;
    for (int l = 0; l < lanes; ++l) acc.push_back({addr + l * stride, bytes});
    const uint64_t s = check_first_lane_form(acc, who);
    if (s > rep.first_lane_span) rep.first_lane_span = s;
    ++rep.waves;
}

// ---------------------------------------------------------------- tensor-major copy

// Waves of one workgroup of tensor t, with the kernel's index map.
void tensor_major_workgroup(const zero_plan* plan, int t, int64_t blk, const uint64_t* bufs,
                            uint64_t dst, Report& rep) {
    using namespace zero::copy;
    const int64_t numel = plan->numels[t];
    const int64_t chunk = plan->chunk_elems[t];
    const int64_t soff = plan->offsets[t];
    const int64_t e0 = blk * kChunk;
    const WorkgroupStart ws = workgroup_start(e0, chunk);
    const bool big = chunk >= kChunk;
    if (ws.r0 != e0 / chunk || ws.local0 != e0 % chunk) fail("workgroup_start disagrees with e0 / chunk");
    for (int v = 0; v < kVecs; ++v) {
        for (int wave = 0; wave < kThreads / 64; ++wave) {
            std::vector<std::pair<uint64_t, uint64_t>> gather_acc, old_acc;
            for (int lane = 0; lane < 64; ++lane) {
                const int64_t tid = wave * 64 + lane;
                const int64_t j = (int64_t(v) * kThreads + tid) * kLane;
                const int64_t e = e0 + j;
                if (!big && e >= numel) break;
                const LanePlace pl = lane_place(ws, chunk, j, big);
                const uint64_t buf = bufs[pl.rank] + 2 * static_cast<uint64_t>(soff + pl.within);
                const uint64_t ten = dst + 2 * static_cast<uint64_t>(e);
                const bool whole = lane_whole(e, numel, pl.within, chunk, buf, ten);
                // every element of the lane: the kernel's place against the definition
                for (int k = 0; k < kLane && e + k < numel; ++k) {
                    int64_t rank, within;
                    if (whole) {
                        rank = pl.rank;
                        within = pl.within + k;
                    } else if (big) {        // the element loop's map
                        const int64_t lk = ws.local0 + j + k;
                        rank = lk < chunk ? ws.r0 : ws.r0 + 1;
                        within = lk < chunk ? lk : lk - chunk;
                    } else {
                        const uint32_t lk = static_cast<uint32_t>(ws.local0 + j) + static_cast<uint32_t>(k);
                        const uint32_t qk = lk / static_cast<uint32_t>(chunk);
                        rank = ws.r0 + static_cast<int64_t>(qk);
                        within = static_cast<int64_t>(lk - qk * static_cast<uint32_t>(chunk));
                    }
                    if (rank != (e + k) / chunk || within != (e + k) % chunk) {
                        fail("element " + std::to_string(e + k) + " of tensor " + std::to_string(t) +
                             " is placed wrongly");
                        return;
                    }
                    if (rank >= plan->n_ranks || soff + within >= plan->shard) {
                        fail("element outside its rank buffer");
                        return;
                    }
                    ++rep.elems_checked;
                }
                if (!whole) continue;
                // gather: one tensor, the first-lane form
                gather_acc.push_back({ten, 2 * kLane});
                // flatten: large chunks store through the rank's own base, small chunks globally
                if (big) {
                    const uint64_t base = bufs[pl.rank] + 2 * static_cast<uint64_t>(soff);
                    const uint64_t off = 2 * static_cast<uint64_t>(pl.within);
                    if (base + off != buf) fail("st_stream_at address differs from the element's");
                    if (off + 2 * kLane > kMaxOff) fail("st_stream_at offset past 2^32");
                    if (off + 2 * kLane > rep.at_max_end) rep.at_max_end = off + 2 * kLane;
                }
                old_acc.push_back({buf, 2 * kLane});
            }
            const uint64_t s = check_first_lane_form(gather_acc, "tensor-major gather");
            if (s > rep.first_lane_span) rep.first_lane_span = s;
            if (!old_acc.empty()) {
                const uint64_t first = old_acc[0].first;
                for (const auto& a : old_acc) {
                    const uint64_t d = a.first > first ? a.first - first + a.second : first - a.first;
                    if (d > rep.old_form_span) rep.old_form_span = d;
                }
            }
            ++rep.waves;
        }
    }
}

void tensor_major(const zero_plan* plan, Report& rep) {
    using namespace zero::copy;
    std::vector<uint64_t> bufs(static_cast<size_t>(plan->n_ranks));
    for (int32_t r = 0; r < plan->n_ranks; ++r)
        bufs[static_cast<size_t>(r)] = kFlatBase + 2 * static_cast<uint64_t>(r) * static_cast<uint64_t>(plan->shard);
    uint64_t dst = kTensorBase;
    for (size_t t = 0; t < plan->numels.size(); ++t) {
        const int64_t n = plan->numels[t];
        if (n <= 0) continue;
        const int64_t chunk = plan->chunk_elems[t];
        const int64_t blocks = (n + kChunk - 1) / kChunk;
        std::vector<int64_t> todo = {0, blocks - 1};
        if (chunk < kChunk) {
            todo.clear();
            for (int64_t b = 0; b < blocks; ++b) todo.push_back(b);
        } else {
            // every workgroup holding a rank boundary, and its neighbours
            for (int64_t r = 1; r * chunk < n; ++r) {
                const int64_t b = r * chunk / kChunk;
                for (int64_t d = -1; d <= 1; ++d)
                    if (b + d >= 0 && b + d < blocks) todo.push_back(b + d);
            }
        }
        for (const int64_t b : todo)
            tensor_major_workgroup(plan, static_cast<int>(t), b, bufs.data(), dst, rep);
        dst += (2 * static_cast<uint64_t>(n) + 255) / 256 * 256;
        if (g_fail) return;
    }
}

// ---------------------------------------------------------------- contiguous kernels

// adamw_kernel<1> on n elements (launches of kMaxBlocks workgroups): lane tid of
// a launch at element off stores P/M/V[off + tid] (4 bytes) and O[off + tid] (2 bytes).
void adamw_flat(int64_t n, Report& rep) {
    constexpr int64_t kMaxBlocks = (int64_t(1) << 32) / 256 - 1;
    const int64_t per_launch = kMaxBlocks * 256;
    for (int64_t off = 0; off < n; off += per_launch) {
        const int64_t len = n - off < per_launch ? n - off : per_launch;
        const int64_t waves = (len + 63) / 64;
        for (const int64_t w : {int64_t(0), waves - 1}) {
            const int lanes = static_cast<int>(len - 64 * w < 64 ? len - 64 * w : 64);
            const int64_t i = off + 64 * w;
            for (int a = 0; a < 3; ++a)
                check_run(kStateBase + a * (uint64_t(1) << 40) + 4 * static_cast<uint64_t>(i), lanes, 4, 4,
                          "adamw fp32", rep);
            check_run(kFlatBase + 2 * static_cast<uint64_t>(i), lanes, 2, 2, "adamw bf16", rep);
        }
    }
}

// The multi-tensor AdamW (list and table): a workgroup's lanes store elements
// base + k * 256 + tid of one tensor, k < 2.
void adamw_multi(int64_t n, Report& rep) {
    const int64_t blocks = (n + 511) / 512;
    for (const int64_t b : {int64_t(0), blocks - 1})
        for (int k = 0; k < 2; ++k)
            for (int w = 0; w < 4; ++w) {
                const int64_t i = b * 512 + k * 256 + w * 64;
                if (i >= n) continue;
                const int lanes = static_cast<int>(n - i < 64 ? n - i : 64);
                check_run(kStateBase + 4 * static_cast<uint64_t>(i), lanes, 4, 4, "multi-tensor adamw", rep);
            }
}

// reduce_vec: lane i (grid-stride, consecutive lanes consecutive i) stores 16
// bytes at out + 16 i; reduce_pass (W = 1): 4 bytes at out + 4 i.
void reduce(int64_t n, Report& rep) {
    const int64_t groups = n / 8;
    if (groups > 0) {
        check_run(kFlatBase, static_cast<int>(groups < 64 ? groups : 64), 16, 16, "reduce_vec", rep);
        const int64_t last = (groups - 1) / 64 * 64;
        check_run(kFlatBase + 16 * static_cast<uint64_t>(last), static_cast<int>(groups - last), 16, 16,
                  "reduce_vec", rep);
    }
    const int64_t units = n / 2;
    if (units > 0) {
        const int64_t last = (units - 1) / 64 * 64;
        check_run(kFlatBase + 4 * static_cast<uint64_t>(last), static_cast<int>(units - last), 4, 4,
                  "reduce_pass", rep);
    }
}

// copy_chunk (segment and copy-table kernels): a workgroup copies one piece's
// chunk; lane i stores 16 bytes at dst + head + 16 i.
void piece_copies(const zero_plan* plan, Report& rep) {
    for (const zero_segment& s : plan->all) {
        const int64_t body = s.length / 8;
        if (body == 0) continue;
        const int64_t last = (body - 1) / 64 * 64;
        const uint64_t dst = kTensorBase + 2 * static_cast<uint64_t>(s.tensor_offset);
        check_run(dst, static_cast<int>(body < 64 ? body : 64), 16, 16, "piece copy", rep);
        check_run(dst + 16 * static_cast<uint64_t>(last), static_cast<int>(body - last), 16, 16, "piece copy", rep);
    }
}

}  // namespace

int main() {
    char word[16];
    int kind, n_ranks, align, n_tensors;
    int plans = 0;
    while (scanf("%15s %d %d %d %d", word, &kind, &n_ranks, &align, &n_tensors) == 5) {
        if (strcmp(word, "plan") != 0) {
            printf("FAIL bad input\n");
            return 1;
        }
        std::vector<int64_t> numels(static_cast<size_t>(n_tensors)), dim0(static_cast<size_t>(n_tensors));
        for (int t = 0; t < n_tensors; ++t)
            if (scanf("%" SCNd64 " %" SCNd64, &numels[static_cast<size_t>(t)], &dim0[static_cast<size_t>(t)]) != 2) {
                printf("FAIL bad tensor line\n");
                return 1;
            }
        zero_plan* plan = nullptr;
        const zero_status st = kind == 1
            ? zero_partition_plan_shard0(numels.data(), dim0.data(), n_tensors, n_ranks, align, &plan)
            : zero_partition_plan(numels.data(), n_tensors, n_ranks, align, &plan);
        if (st != ZERO_OK) {
            printf("FAIL plan: %s\n", zero_last_error());
            return 1;
        }
        Report rep;
        const bool tm = zero::copy::fits_tensor_major(plan);
        if (tm) tensor_major(plan, rep);
        piece_copies(plan, rep);       // flat plans, and the gaps and tables of Shard(0) plans
        adamw_flat(plan->shard, rep);
        reduce(plan->shard, rep);
        for (const int64_t n : plan->numels)
            if (n > 0) adamw_multi(n, rep);
        printf("plan %d kind=%d ranks=%d S=%" PRId64 " route=%s waves=%" PRId64 " elems=%" PRId64
               " first_lane_span=%" PRIu64 " at_max_end=%" PRIu64 " old_form_span=%" PRIu64 "\n",
               plans, kind, n_ranks, plan->shard,
               tm ? (zero::copy::fits_compact(plan) ? "tensor-major-compact" : "tensor-major-wide")
                  : "segments",
               rep.waves, rep.elems_checked, rep.first_lane_span, rep.at_max_end, rep.old_form_span);
        zero_plan_free(plan);
        ++plans;
        if (g_fail) return 1;
    }
    printf("ok\n");
    return 0;
}
