// Host check of the device tables' per-workgroup index layout (internal.hpp):
// a launch of nb workgroups reads entry b0 + (x % 8) * ceil(nb / 8) + x / 8 for
// its workgroup x. Every entry read must hold that workgroup's value, and lie
// inside the index, for table sizes around the launch boundaries.
#include <cstdio>
#include <random>

#include "internal.hpp"

int main() {
    std::mt19937_64 rng(7);
    const int64_t L = zero::kTableLaunchBlocks;
    if (L % 8 != 0 || L * 256 >= (int64_t(1) << 32)) {
        printf("bad launch size %lld\n", static_cast<long long>(L));
        return 1;
    }
    const int64_t totals[] = {1, 7, 8, 9, 15, 16, 17, 255, 60762, 1000003, L - 1, L, L + 1, 2 * L + 5};
    for (const int64_t total : totals) {
        std::vector<uint32_t> plain(static_cast<size_t>(total));
        for (auto& v : plain) v = static_cast<uint32_t>(rng());
        const std::vector<uint32_t> idx = zero::xcd_major_index(plain);
        if (idx.size() != plain.size() + 7) {
            printf("size mismatch at %lld\n", static_cast<long long>(total));
            return 1;
        }
        for (int64_t b0 = 0; b0 < total; b0 += L) {
            const int64_t nb = total - b0 < L ? total - b0 : L;
            const int64_t per = (nb + 7) / 8;
            for (int64_t x = 0; x < nb; ++x) {
                const int64_t e = b0 + (x & 7) * per + (x >> 3);
                if (e >= static_cast<int64_t>(idx.size()) || idx[static_cast<size_t>(e)] != plain[static_cast<size_t>(b0 + x)]) {
                    printf("wrong entry: total %lld, launch at %lld, workgroup %lld\n",
                           static_cast<long long>(total), static_cast<long long>(b0), static_cast<long long>(x));
                    return 1;
                }
            }
        }
    }
    printf("ok\n");
    return 0;
}
