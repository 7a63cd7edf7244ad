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
// `pair` (one chunk per XCD, every item resident in one round, two workgroups
// per CU or one): the second half of the XCD's list is taken in reverse, so
// the workgroups that fill a CU's slots in the second pass over the CUs get
// the light items and each CU a like share of heavy and light causal tiles.
__device__ __forceinline__ int dealt_item(int w, int chunk, int nitems, int pair) {
    const int x = w % kXcds;
    int s = w / kXcds;
    if (pair) {
        const int n = min(chunk, nitems - x * chunk);
        const int H = (n + 1) / 2;
        if (s >= H && s < n) s = H + (n - 1 - s);
    }
    const int k = s / chunk;
    const int c = kXcds * k + ((k & 1) ? kXcds - 1 - x : x);
    const long long item = (long long)c * chunk + s % chunk;
    return item < nitems ? (int)item : -1;
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
