// Host check of the work deal (deal.h): for each launch shape, every work
// item of the list is taken by exactly one workgroup of the grid, for the
// chunked snake deal, the one-round weight deal and the several-round weight
// deal. Prints one line per shape and exits non-zero on the first failure.
#include "deal.h"

#include <cstdio>
#include <vector>

namespace {

// the arguments the launchers pass: (batch, kv head) groups of G heads x nqt
// query tiles, `slots` workgroups per CU
int check(long long B, long long Hq, long long Hkv, long long nqt, bool paged, int causal, int num_cu, int slots) {
    const long long nitems = B * Hq * nqt;
    const int G = (int)(Hq / Hkv);
    const attn::Deal deal = attn::make_deal(nitems, (long long)G * nqt, G, paged);
    const int bal = paged ? 0 : attn::balance_arg(nitems, deal.chunk, (long long)G * nqt, deal.grid, causal, num_cu, slots);
    std::vector<int> seen((size_t)nitems, 0);
    for (long long w = 0; w < deal.grid; ++w) {
        const int item = attn::dealt_item((int)w, (int)deal.chunk, (int)nitems, bal, (int)nqt, G);
        if (item < -1 || item >= nitems) {
            std::printf("FAIL B=%lld Hq=%lld Hkv=%lld nqt=%lld paged=%d: workgroup %lld -> item %d\n", B, Hq, Hkv, nqt,
                        (int)paged, w, item);
            return 1;
        }
        if (item >= 0) ++seen[(size_t)item];
    }
    for (long long i = 0; i < nitems; ++i)
        if (seen[(size_t)i] != 1) {
            std::printf("FAIL B=%lld Hq=%lld Hkv=%lld nqt=%lld paged=%d: item %lld taken %d times\n", B, Hq, Hkv, nqt,
                        (int)paged, i, seen[(size_t)i]);
            return 1;
        }
    std::printf("ok B=%lld Hq=%lld Hkv=%lld nqt=%lld paged=%d causal=%d cu=%d slots=%d: chunk %lld grid %lld bal %d\n", B,
                Hq, Hkv, nqt, (int)paged, causal, num_cu, slots, deal.chunk, deal.grid, bal);
    return 0;
}

}  // namespace

int main() {
    const long long shapes[][4] = {
        // B, Hq, Hkv, nqt
        {4, 32, 8, 16},  {8, 12, 12, 8},  {16, 12, 12, 8}, {32, 12, 12, 8}, {2, 16, 16, 16}, {12, 32, 8, 8},
        {1, 8, 1, 64},   {1, 32, 8, 64},  {1, 16, 16, 16}, {3, 6, 3, 3},    {5, 6, 3, 1},    {1, 1, 1, 1},
        {600, 8, 2, 1},  {7, 9, 3, 5},    {2, 4, 2, 11},   {64, 32, 8, 1},  {4, 16, 16, 32}, {1, 24, 8, 13},
    };
    for (const auto& s : shapes)
        for (int paged = 0; paged < 2; ++paged)
            for (int causal = 0; causal < 2; ++causal)
                for (int slots : {1, 2, 3})
                    for (int cu : {256, 240})
                        if (check(s[0], s[1], s[2], s[3], paged != 0, causal, cu, slots)) return 1;
    std::printf("all shapes ok\n");
    return 0;
}
