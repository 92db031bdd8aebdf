// Host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer
// (built with g++ by tests/test_host_sanitizers_cpu.py): the planner
// (plan.cpp), the copy piece lists and copy-table contents (pieces.cpp), the
// per-workgroup index (internal.hpp) and the tensor-major routing
// (tensor_major.hpp). Every call's results are checked against the layout's
// definition, so the run is both a sanitizer pass and a consistency check:
//   - flat plans: P a multiple of N_d * A, every element of [0, Phi) in exactly
//     one segment at rank g / S, offset g % S;
//   - Shard(0) plans: every element of every tensor in exactly one segment, at
//     rank row / chunk_rows;
//   - gather pieces: each tensor covered exactly once; flatten pieces: [0, P)
//     covered exactly once, gaps zero-filled;
//   - copy-table contents: every workgroup's descriptor is the piece it copies;
//   - argument errors and sizes that overflow int64 return their status codes.
// Input (stdin): as tests/host_store_span.cpp ("plan <kind> <n_ranks> <align>
// <T>" then T lines "<numel> <dim0>"), followed by random lists drawn here.
// Prints "ok" or lines starting "FAIL".
#include <cinttypes>
#include <climits>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "internal.hpp"
#include "pieces.hpp"
#include "schedule.hpp"
#include "tensor_major.hpp"

namespace {

int g_fail = 0;
void fail(const std::string& what) {
    if (g_fail++ < 20) printf("FAIL %s\n", what.c_str());
}

// Fake 256-byte-aligned device addresses: the checks compare addresses only.
uint16_t* fake(uint64_t base) { return reinterpret_cast<uint16_t*>(static_cast<uintptr_t>(base)); }

// Reduce-table contents for every rank: the pieces tile [0, S) in shard order,
// the tensor pieces are exactly the rank's segments, the 16-byte flag follows
// its rule, every workgroup's index entry names the piece its chunk lies in,
// the replica pointers are tensor-major; a NULL tensor a segment needs, and a
// shard_grad overlapping a replica tensor, are refused.
void check_reduce_table(const zero_plan* p, const std::vector<int64_t>& numels, int n_ranks) {
    const int64_t T = static_cast<int64_t>(numels.size());
    const int64_t S = zero_plan_shard_numel(p);
    const int32_t R = 3;
    const int64_t chunk = 2048;
    // replica k's tensor t at a 16-byte-aligned fake address, except replica 1's odd tensors
    std::vector<const uint16_t*> reps(static_cast<size_t>(R * T));
    for (int32_t k = 0; k < R; ++k)
        for (int64_t t = 0; t < T; ++t)
            reps[static_cast<size_t>(k * T + t)] =
                fake((uint64_t(k + 1) << 44) + (uint64_t(t) << 36) + (k == 1 && t % 2 == 1 ? 2 : 0));
    const uint16_t* grad = fake(uint64_t(7) << 44);
    for (int r = 0; r < n_ranks; ++r) {
        std::vector<zero::copy::RPieceDesc> descs;
        std::vector<uint32_t> index;
        std::vector<const uint16_t*> ptrs;
        int64_t blocks = -1;
        if (zero::copy::reduce_table_contents(p, r, reps.data(), R, grad, chunk, &descs, &index, &ptrs,
                                              &blocks, "t") != ZERO_OK) {
            fail("reduce table contents");
            return;
        }
        for (int64_t t = 0; t < T; ++t)
            for (int32_t k = 0; k < R; ++k)
                if (ptrs[static_cast<size_t>(t * R + k)] != reps[static_cast<size_t>(k * T + t)])
                    fail("replica pointers tensor-major");
        const int32_t ns = zero_plan_num_segments(p, r);
        std::vector<zero_segment> segs(static_cast<size_t>(ns) + 1);
        int32_t count = 0;
        if (zero_plan_segments(p, r, segs.data(), ns, &count) != ZERO_OK) fail("segments");
        int64_t pos = 0, blocks_seen = 0;
        int32_t seg_i = 0;
        for (const auto& d : descs) {
            if (d.dst_off != pos || d.len <= 0) { fail("reduce pieces tile the shard"); return; }
            if (d.first_block != blocks_seen) fail("reduce piece first block");
            blocks_seen += (d.len + chunk - 1) / chunk;
            if (d.tensor >= 0) {
                if (seg_i >= count) { fail("more tensor pieces than segments"); return; }
                const zero_segment& sg = segs[static_cast<size_t>(seg_i++)];
                if (sg.tensor != d.tensor || sg.tensor_offset != d.src_off || sg.shard_offset != d.dst_off ||
                    sg.length != d.len)
                    fail("tensor piece is the rank's segment");
                const bool aligned = !(d.tensor % 2 == 1);     // replica 1's odd tensors are 2 bytes off
                const bool want = aligned && d.src_off % 8 == 0 && d.dst_off % 8 == 0;
                if ((d.vec != 0) != want) fail("16-byte flag");
            } else if (d.vec != 0) {
                fail("padding pieces take no 16-byte path");
            }
            pos = d.dst_off + d.len;
        }
        if (pos != S || seg_i != count) fail("reduce pieces cover S and every segment");
        if (blocks != blocks_seen) fail("reduce table blocks");
        for (int64_t b0 = 0; b0 < blocks; b0 += zero::kTableLaunchBlocks) {
            const int64_t nb = blocks - b0 < zero::kTableLaunchBlocks ? blocks - b0 : zero::kTableLaunchBlocks;
            const int64_t per = (nb + 7) / 8;
            for (int64_t x = 0; x < nb; ++x) {
                const size_t e = static_cast<size_t>(b0 + (x & 7) * per + (x >> 3));
                if (e >= index.size() || index[e] >= descs.size()) { fail("reduce index out of range"); return; }
                const auto& d = descs[index[e]];
                const int64_t start = (b0 + x - d.first_block) * chunk;
                if (start < 0 || start >= d.len) { fail("reduce workgroup outside its piece"); return; }
            }
        }
        if (count > 0) {              // errors: a needed tensor missing; the output over a tensor
            const int32_t t = segs[0].tensor;
            std::vector<const uint16_t*> bad = reps;
            bad[static_cast<size_t>(2 * T + t)] = nullptr;
            if (zero::copy::reduce_table_contents(p, r, bad.data(), R, grad, chunk, &descs, &index, &ptrs,
                                                  &blocks, "t") != ZERO_EINVAL)
                fail("NULL needed replica tensor");
            if (zero::copy::reduce_table_contents(p, r, reps.data(), R, reps[static_cast<size_t>(t)], chunk,
                                                  &descs, &index, &ptrs, &blocks, "t") != ZERO_EINVAL)
                fail("shard_grad over a replica tensor");
        }
    }
}

void check_plan(const zero_plan* p, const std::vector<int64_t>& numels, const std::vector<int64_t>& dim0,
                int kind, int n_ranks, int align, bool deep) {
    const int T = static_cast<int>(numels.size());
    if (zero_plan_num_tensors(p) != T || zero_plan_num_ranks(p) != n_ranks || zero_plan_kind(p) != kind)
        fail("plan queries");
    const int64_t S = zero_plan_shard_numel(p), P = zero_plan_padded_numel(p);
    if (P != S * n_ranks || S % align != 0) fail("P = N_d * S, S a multiple of A");
    int64_t phi = 0;
    for (int64_t n : numels) phi += n;
    if (zero_plan_numel(p) != phi) fail("Phi");
    if (zero_plan_tensor_offset(p, -1) != -1 || zero_plan_tensor_offset(p, T) != -1 ||
        zero_plan_tensor_numel(p, T) != -1 || zero_plan_num_segments(p, n_ranks) != -1 ||
        zero_plan_num_segments(p, -1) != -1)
        fail("out-of-range queries return -1");
    for (int stage = -1; stage <= 4; ++stage)
        for (int padded = 0; padded < 2; ++padded) {
            double b = -1;
            const zero_status st = zero_plan_memory_bytes(p, stage, padded, &b);
            if ((stage >= 0 && stage <= 3) != (st == ZERO_OK)) fail("memory_bytes stage check");
        }
    // segments, per rank, through the ABI
    std::vector<zero_segment> all;
    for (int r = 0; r < n_ranks; ++r) {
        const int32_t n = zero_plan_num_segments(p, r);
        int32_t count = -1;
        if (n > 0) {
            std::vector<zero_segment> tiny(static_cast<size_t>(n - 1) + 1);
            if (zero_plan_segments(p, r, tiny.data(), n - 1, &count) != ZERO_ENOSPACE || count != n)
                fail("segments: capacity too small");
        }
        std::vector<zero_segment> segs(static_cast<size_t>(n) + 1);
        if (zero_plan_segments(p, r, segs.data(), n, &count) != ZERO_OK || count != n) fail("segments");
        for (int i = 0; i < n; ++i) {
            const zero_segment& s = segs[static_cast<size_t>(i)];
            if (s.rank != r || s.length <= 0 || s.shard_offset < 0 || s.shard_offset + s.length > S ||
                s.tensor < 0 || s.tensor >= T || s.tensor_offset < 0 ||
                s.tensor_offset + s.length > numels[static_cast<size_t>(s.tensor)])
                fail("segment out of range");
            all.push_back(s);
        }
    }
    if (!deep) return;
    // every tensor element in exactly one segment, at its place by definition
    std::vector<std::vector<uint8_t>> seen(static_cast<size_t>(T));
    for (int t = 0; t < T; ++t) seen[static_cast<size_t>(t)].assign(static_cast<size_t>(numels[static_cast<size_t>(t)]), 0);
    int64_t off = 0;
    std::vector<int64_t> offs(static_cast<size_t>(T));
    for (int t = 0; t < T; ++t) { offs[static_cast<size_t>(t)] = off; off += numels[static_cast<size_t>(t)]; }
    for (const zero_segment& s : all)
        for (int64_t k = 0; k < s.length; ++k) {
            const int64_t e = s.tensor_offset + k;
            uint8_t& v = seen[static_cast<size_t>(s.tensor)][static_cast<size_t>(e)];
            if (v) { fail("element covered twice"); return; }
            v = 1;
            if (kind == 0) {
                const int64_t g = offs[static_cast<size_t>(s.tensor)] + e;
                if (g / S != s.rank || g % S != s.shard_offset + k) { fail("flat place"); return; }
            } else {
                const int64_t rows = dim0[static_cast<size_t>(s.tensor)];
                const int64_t inner = numels[static_cast<size_t>(s.tensor)] / rows;
                const int64_t c = rows / n_ranks + (rows % n_ranks != 0);
                if ((e / inner) / c != s.rank ||
                    s.shard_offset + k != zero_plan_tensor_offset(p, s.tensor) + (e - s.rank * c * inner)) {
                    fail("Shard(0) place");
                    return;
                }
            }
        }
    for (int t = 0; t < T; ++t)
        for (uint8_t v : seen[static_cast<size_t>(t)])
            if (!v) { fail("element not covered"); return; }

    // piece lists with fake addresses: tensors far apart, the flat buffer, the shards
    std::vector<uint16_t*> tensors(static_cast<size_t>(T)), shards(static_cast<size_t>(n_ranks));
    const uint64_t tbase = 0x100000000000ull, fbase = 0x200000000000ull;
    for (int t = 0; t < T; ++t) tensors[static_cast<size_t>(t)] = fake(tbase + (static_cast<uint64_t>(t) << 36));
    for (int r = 0; r < n_ranks; ++r) shards[static_cast<size_t>(r)] = fake(fbase) + static_cast<int64_t>(r) * S;
    // disjoint buffers pass the range checks; a tensor moved onto the last rank's shard does not
    if (zero::copy::check_gather_ranges(p, shards.data(), tensors.data(), "t") != ZERO_OK ||
        zero::copy::check_flatten_ranges(p, tensors.data(), fake(fbase), "t") != ZERO_OK)
        fail("range checks refuse disjoint buffers");
    for (int t = 0; t < T; ++t) {
        if (p->numels[static_cast<size_t>(t)] == 0 || S == 0) continue;
        std::vector<uint16_t*> moved = tensors;
        moved[static_cast<size_t>(t)] = shards[static_cast<size_t>(n_ranks - 1)] + S - 1;
        if (zero::copy::check_gather_ranges(p, shards.data(), moved.data(), "t") != ZERO_EINVAL ||
            zero::copy::check_flatten_ranges(p, moved.data(), fake(fbase), "t") != ZERO_EINVAL)
            fail("range checks miss a tensor over a shard");
        break;
    }
    const std::vector<zero::copy::Piece> g = zero::copy::gather_pieces(p, shards.data(), tensors.data());
    int64_t gathered = 0;
    for (const auto& pc : g) gathered += pc.len;
    if (gathered != phi) fail("gather pieces cover Phi");
    for (int with = 0; with < 2; ++with) {
        const auto f = zero::copy::flatten_pieces(p, tensors.data(), fake(fbase), with != 0);
        std::vector<uint8_t> cov(static_cast<size_t>(P), 0);
        for (const auto& pc : f) {
            const int64_t at = pc.dst - fake(fbase);
            if (at < 0 || pc.len <= 0 || at + pc.len > P) { fail("flatten piece out of range"); return; }
            for (int64_t k = 0; k < pc.len; ++k) {
                if (cov[static_cast<size_t>(at + k)]) { fail("flatten covers twice"); return; }
                cov[static_cast<size_t>(at + k)] = 1;
            }
        }
        int64_t covered = 0;
        for (uint8_t v : cov) covered += v;
        if (with && covered != P) fail("flatten pieces cover P");
        if (!with && covered != P - phi) fail("flatten gaps are P - Phi");
        // copy-table contents: workgroup b's descriptor holds the chunk it copies
        std::vector<zero::copy::PieceDesc> descs;
        std::vector<uint32_t> index;
        int64_t blocks = -1;
        if (zero::copy::copy_table_contents(f, zero::copy::kChunk, &descs, &index, &blocks, "t") != ZERO_OK)
            fail("copy table contents");
        for (int64_t b0 = 0; b0 < blocks; b0 += zero::kTableLaunchBlocks) {
            const int64_t nb = blocks - b0 < zero::kTableLaunchBlocks ? blocks - b0 : zero::kTableLaunchBlocks;
            const int64_t per = (nb + 7) / 8;
            for (int64_t x = 0; x < nb; ++x) {
                const size_t e = static_cast<size_t>(b0 + (x & 7) * per + (x >> 3));
                if (e >= index.size() || index[e] >= descs.size()) { fail("index out of range"); return; }
                const auto& d = descs[index[e]];
                const int64_t start = (b0 + x - d.first_block) * zero::copy::kChunk;
                if (start < 0 || start >= d.len) { fail("workgroup outside its piece"); return; }
            }
        }
    }
    (void)zero::copy::fits_tensor_major(p);
    (void)zero::copy::fits_compact(p);
    check_reduce_table(p, numels, n_ranks);
}

bool run_plan(int kind, int n_ranks, int align, const std::vector<int64_t>& numels,
              const std::vector<int64_t>& dim0, bool deep) {
    zero_plan* p = nullptr;
    const int T = static_cast<int>(numels.size());
    const zero_status st = kind == 1
        ? zero_partition_plan_shard0(numels.data(), dim0.data(), T, n_ranks, align, &p)
        : zero_partition_plan(numels.data(), T, n_ranks, align, &p);
    if (st != ZERO_OK) return false;
    check_plan(p, numels, dim0, kind, n_ranks, align, deep);
    zero_plan_free(p);
    return true;
}

void edge_cases() {
    zero_plan* p = nullptr;
    const int64_t big[] = {INT64_MAX - 5, 7};
    const int64_t one[] = {1, 1};
    if (zero_partition_plan(big, 2, 1, 1, &p) != ZERO_ERANGE || p) fail("flat: total overflows");
    if (zero_partition_plan(big, 1, 3, 128, &p) != ZERO_ERANGE || p) fail("flat: padding overflows");
    if (zero_partition_plan_shard0(big, one, 1, 1, 128, &p) != ZERO_ERANGE || p)
        fail("Shard(0): alignment overflows");
    const int64_t rows_big[] = {INT64_MAX - 1};
    const int64_t d_big[] = {INT64_MAX - 1};
    if (zero_partition_plan_shard0(rows_big, d_big, 1, 64, 1, &p) == ZERO_OK) {
        // rows near INT64_MAX: the rank cut must not overflow
        int32_t count = -1;
        zero_segment seg;
        for (int r = 0; r < 64; ++r) (void)zero_plan_segments(p, r, &seg, 1, &count);
        zero_plan_free(p);
        p = nullptr;
    }
    const int64_t neg[] = {-1};
    if (zero_partition_plan(neg, 1, 1, 1, &p) != ZERO_EINVAL) fail("negative numel");
    if (zero_partition_plan(one, 1, 0, 1, &p) != ZERO_EINVAL) fail("n_ranks 0");
    if (zero_partition_plan(one, 1, 1, 0, &p) != ZERO_EINVAL) fail("align 0");
    if (zero_partition_plan(nullptr, 1, 1, 1, &p) != ZERO_EINVAL) fail("NULL numels");
    if (zero_partition_plan(one, 1, 1, 1, nullptr) != ZERO_EINVAL) fail("NULL out");
    const int64_t nd[] = {10}, bad_d0[] = {3};
    if (zero_partition_plan_shard0(nd, bad_d0, 1, 2, 1, &p) != ZERO_EINVAL) fail("dim0 must divide");
    if (zero_plan_segments(nullptr, 0, nullptr, 0, nullptr) != ZERO_EINVAL) fail("NULL plan segments");
    if (zero_plan_numel(nullptr) != -1 || zero_plan_kind(nullptr) != -1) fail("NULL queries");
    zero_plan_free(nullptr);
    // empty lists and zero-sized tensors
    if (!run_plan(0, 3, 128, {}, {}, true)) fail("empty flat plan");
    if (!run_plan(1, 3, 128, {}, {}, true)) fail("empty Shard(0) plan");
    if (!run_plan(0, 4, 8, {0, 5, 0}, {0, 5, 0}, true)) fail("zero-sized flat");
    if (!run_plan(1, 4, 8, {0, 6, 0}, {0, 2, 0}, true)) fail("zero-sized Shard(0)");
}

// The sorted overlap check against the pairwise one on random lists of small
// ranges (many touching, some empty or NULL): both find a clash on the same
// lists, and a clash the sorted one names is a real one.
void check_overlap_search() {
    std::mt19937_64 rng(5);
    int clashes = 0;
    for (int it = 0; it < 20000; ++it) {
        const int nw = static_cast<int>(rng() % 7), nr = static_cast<int>(rng() % 5);
        std::vector<zero::Span> wr, rd;
        auto one = [&](const char* name, int i) {
            const uint64_t at = 0x1000 + 8 * (rng() % 40);
            const size_t bytes = 8 * (rng() % 6);            // 0 .. 40 bytes
            const bool null = rng() % 16 == 0;
            return zero::Span{null ? nullptr : fake(at), bytes, name, i};
        };
        for (int i = 0; i < nw; ++i) wr.push_back(one("w", i));
        for (int i = 0; i < nr; ++i) rd.push_back(one("r", i));
        auto live = [](std::vector<zero::Span> v) {
            for (auto& x : v)
                if (x.p == nullptr) x.bytes = 0;
            return v;
        };
        const std::vector<zero::Span> lw = live(wr), lr = live(rd);
        const std::string brute = zero::first_overlap(lw.data(), nw, lr.data(), nr);
        const std::string sorted = zero::copy::first_overlap_sorted(wr, rd);
        if (brute.empty() != sorted.empty()) {
            fail("sorted overlap search: '" + sorted + "' against '" + brute + "'");
            return;
        }
        if (sorted.empty()) continue;
        ++clashes;
        // the named pair overlaps
        auto find = [&](const std::string& name) -> const zero::Span* {
            for (const auto& x : lw)
                if (zero::span_name(x) == name) return &x;
            for (const auto& x : lr)
                if (zero::span_name(x) == name) return &x;
            return nullptr;
        };
        const size_t cut = sorted.find(" overlaps ");
        const zero::Span* a = find(sorted.substr(0, cut));
        const zero::Span* b = find(sorted.substr(cut + 10));
        if (!a || !b || !zero::ranges_overlap(a->p, a->bytes, b->p, b->bytes)) fail("named pair: " + sorted);
    }
    if (clashes < 1000) fail("too few overlapping lists drawn");
}

// A step schedule's table against the direct per-step computation: entry t - 1
// is step t's scalars (with lr[min(t, n) - 1]), and every step past the table
// has the last entry's scalars, bit for bit.
void check_schedules() {
    struct Case { std::vector<double> lr; double b1, b2, eps, wd; };
    const Case cases[] = {{{1e-3}, 0.9, 0.999, 1e-8, 0.01},
                          {{1e-3, 2e-3, 3e-3, 2.5e-3}, 0.9, 0.99, 1e-8, 0.1},
                          {{0.5}, 0.0, 0.0, 1e-6, 0.0},
                          {{1e-4}, 0.99, 0.9999, 1.0, -0.5},
                          {std::vector<double>(50000, 7e-4), 0.5, 0.9, 1e-8, 0.01}};
    for (const Case& c : cases) {
        std::vector<zero::adam::StepScalars> table;
        if (zero::adam::schedule_table(c.lr.data(), static_cast<int64_t>(c.lr.size()), c.b1, c.b2, c.eps,
                                       c.wd, &table, "t") != ZERO_OK) {
            fail("schedule table refused");
            continue;
        }
        const int64_t L = static_cast<int64_t>(table.size()), n = static_cast<int64_t>(c.lr.size());
        if (L < n) fail("schedule shorter than its learning rates");
        auto same = [](const zero::adam::StepScalars& a, const zero::adam::StepScalars& b) {
            return std::memcmp(&a, &b, sizeof(a)) == 0;
        };
        for (int64_t t = 1; t <= L + 2000; ++t) {
            zero::adam::StepScalars want{};
            if (zero::adam::step_scalars(t, c.lr[static_cast<size_t>((t < n ? t : n) - 1)], c.b1, c.b2, c.wd,
                                         c.eps, &want, "t") != ZERO_OK) {
                fail("step scalars refused");
                break;
            }
            const auto& got = table[static_cast<size_t>((t < L ? t : L) - 1)];
            if (!same(got, want)) { fail("schedule entry differs from the step's scalars"); break; }
        }
        for (const int64_t t : {int64_t(1) << 31, int64_t(1) << 40, int64_t(1) << 62}) {
            zero::adam::StepScalars want{};
            zero::adam::step_scalars(t, c.lr.back(), c.b1, c.b2, c.wd, c.eps, &want, "t");
            if (!same(table.back(), want)) fail("far step differs from the schedule's last entry");
        }
    }
    if (zero::adam::settled_step(0.9, 0.999, zero::adam::kMaxScheduleSteps) != 38797) fail("settled step");
    if (zero::adam::settled_step(0.0, 0.0, 100) != 1) fail("settled step of zero betas");
    if (zero::adam::settled_step(0.9, 1.0 - 1e-7, zero::adam::kMaxScheduleSteps) != -1) fail("settled step cap");
}

}  // namespace

int main() {
    char word[16];
    int kind, n_ranks, align, T;
    while (scanf("%15s %d %d %d %d", word, &kind, &n_ranks, &align, &T) == 5) {
        if (strcmp(word, "plan") != 0) { printf("FAIL bad input\n"); return 1; }
        std::vector<int64_t> numels(static_cast<size_t>(T)), dim0(static_cast<size_t>(T));
        for (int t = 0; t < T; ++t)
            if (scanf("%" SCNd64 " %" SCNd64, &numels[static_cast<size_t>(t)], &dim0[static_cast<size_t>(t)]) != 2) {
                printf("FAIL bad tensor line\n");
                return 1;
            }
        int64_t phi = 0;
        for (int64_t n : numels) phi += n;
        if (!run_plan(kind, n_ranks, align, numels, dim0, phi <= 20000000)) fail("workload plan refused");
    }
    edge_cases();
    check_overlap_search();
    check_schedules();
    std::mt19937_64 rng(11);
    for (int it = 0; it < 400; ++it) {
        const int T = static_cast<int>(rng() % 9);
        const int nr = 1 + static_cast<int>(rng() % 9);
        const int al = (int[]){1, 3, 8, 128}[rng() % 4];
        std::vector<int64_t> numels, dim0;
        for (int t = 0; t < T; ++t) {
            const int64_t rows = static_cast<int64_t>(rng() % 40);
            const int64_t inner = 1 + static_cast<int64_t>(rng() % 50);
            numels.push_back(rows * inner);
            dim0.push_back(rows);
        }
        if (!run_plan(0, nr, al, numels, dim0, true)) fail("random flat plan refused");
        if (!run_plan(1, nr, al, numels, dim0, true)) fail("random Shard(0) plan refused");
        if (g_fail) break;
    }
    if (g_fail) return 1;
    printf("ok\n");
    return 0;
}
