// Work-item deal over the XCDs of an MI355X for the attention kernels whose
// work items are (batch, kv head) groups of query tiles listed heaviest causal
// tile first: which XCD runs which item, and in which order.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

namespace attn {

constexpr int kXcds = 8;   // XCDs of an MI355X; workgroup w is dispatched to XCD w % 8

// Work item of workgroup w under the chunked snake deal (-1: no item). Slot s
// of XCD x = w % 8 is position s % chunk of that XCD's (s / chunk)-th chunk;
// its k-th chunk is the list's chunk 8k + x for even k and 8k + 7 - x for odd k.
//
// `bal` != 0 (one chunk per XCD holding whole groups, causal items): the
// XCD's items are taken by weight rank, query tiles heaviest first (then the
// groups, then the heads of a group), instead of group by group.
//  * bal > 0 (every item resident in one round of dispatch, bal = CUs per
//    XCD): the dispatcher hands the XCD's slots s = 0, 1, ... to its CUs
//    round by round, slot s to CU s % bal, and the ranks run forward over the
//    CUs in even rounds and backward in odd ones, so each CU gets a like mix
//    of heavy and light causal tiles. A partial last round keeps slot order.
//  * bal < 0 (several rounds): slot s takes rank s, so the dispatcher, which
//    gives the next slot to the first CU that frees up, runs the XCD's
//    heaviest items first and ends on its lightest.
__host__ __device__ __forceinline__ int dealt_item(int w, int chunk, int nitems, int bal, int nqt, int G) {
    const int x = w % kXcds;
    const int s = w / kXcds;
    if (bal != 0) {
        const int n = nitems - x * chunk < chunk ? nitems - x * chunk : chunk;   // this XCD's items: whole groups
        if (s >= n) return -1;
        int rank = s;
        if (bal > 0) {
            const int r = s / bal, p = s % bal;
            const bool partial_last = r == (n - 1) / bal && n % bal != 0;
            rank = ((r & 1) && !partial_last) ? r * bal + (bal - 1 - p) : s;
        }
        const int per_tile = n / nqt;                    // groups of this XCD x G
        const int qi = rank / per_tile, rest = rank % per_tile;
        return x * chunk + ((rest / G) * nqt + qi) * G + rest % G;
    }
    const int k = s / chunk;
    const int c = kXcds * k + ((k & 1) ? kXcds - 1 - x : x);
    const long long item = (long long)c * chunk + s % chunk;
    return item < nitems ? (int)item : -1;
}

// `bal` argument of dealt_item for a launch of causal items whose deal is one
// chunk per XCD of whole groups: CUs per XCD when every item is resident at
// once (the grid fits `slots_per_cu` workgroups on each CU); -1 when a group
// fills less than two rounds of the XCD's slots; else 0. Taken group by
// group, the last groups' heaviest tiles would start late (2 x 16 heads x 4096
// tokens: a simulated greedy dispatch ends 46 % after a perfect split); with
// two rounds or more per group that order is as balanced as the weight order
// and keeps fewer groups' K/V in the XCD's L2 at a time (the 4 x 32 heads x
// 4096-token prefill runs 1.5 % faster in it).
inline int balance_arg(long long nitems, long long chunk, long long group_items, long long grid, int causal,
                       int num_cu, int slots_per_cu) {
    const int cus = num_cu > 0 ? num_cu : 256;
    const bool one_chunk_per_xcd = (nitems + chunk - 1) / chunk <= kXcds;
    const bool whole_groups = chunk % group_items == 0;
    if (!(causal && one_chunk_per_xcd && whole_groups && cus % kXcds == 0)) return 0;
    const long long xcd_slots = (long long)(cus / kXcds) * slots_per_cu;
    if (grid <= (long long)cus * slots_per_cu) return cus / kXcds;
    return group_items < 2 * xcd_slots ? -1 : 0;
}

// Host side of the deal: the chunk size and the grid that covers every chunk.
// With at least one (batch, kv head) group per XCD, contiguous K/V takes one
// run of 1/8 of the list per XCD and a paged cache one group per chunk. With
// fewer groups (MQA, a single sequence), a chunk is the G query heads of one
// (group, query tile): with one run per XCD the heaviest query tiles would
// all land on the first XCDs.
struct Deal {
    long long chunk, grid;
};
inline Deal make_deal(long long nitems, long long group_items, int G, bool paged) {
    const long long per_xcd = (nitems + kXcds - 1) / kXcds;
    const long long ngroups = (nitems + group_items - 1) / group_items;
    long long chunk = ngroups < kXcds ? (long long)G : paged ? std::min(group_items, per_xcd) : per_xcd;
    chunk = std::max(1LL, chunk);
    const long long nchunks = (nitems + chunk - 1) / chunk;
    const long long rounds = (nchunks + kXcds - 1) / kXcds;
    return {chunk, rounds * kXcds * chunk};
}

}  // namespace attn
