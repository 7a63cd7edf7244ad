// Index arithmetic of the paged KV cache, shared by the kernels that read or
// write it (decode, paged prefill, KV append) and by the host program that
// replays their accesses (tests/native/paging_check.cpp).
//
// Layout ("LLM 核心技术：Attention 机制的实现与优化", PagedAttention section: the
// cache lives in fixed-size pages of one global pool, reached through a
// per-sequence page table): pools [pages, Hkv, page_size, D]; the page table
// is ragged, sequence b owning ceil(len_b / page_size) consecutive entries
// from off_b = sum over j < b of ceil(len_j / page_size); token t of the
// sequence is slot t % page_size of page table[off_b + t / page_size].
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace attn {

// Page-table entries a sequence of len tokens owns.
__host__ __device__ __forceinline__ int seq_pages(int len, int ps_log2) {
    return (len + (1 << ps_log2) - 1) >> ps_log2;
}

// First visible token of a decode over len cached tokens: a window keeps the
// `window` most recent ones, the current one included (0: every token).
__host__ __device__ __forceinline__ int window_first(int len, int window) {
    return window > 0 && len > window ? len - window : 0;
}

// The blocks of `unit` tokens that hold the visible tokens first .. len - 1,
// cut into nsplit contiguous runs as evenly as whole blocks allow; run
// `split` is blocks [begin, end) (empty when there are fewer blocks than
// runs).
struct UnitRun {
    int begin, end;
};
__host__ __device__ __forceinline__ UnitRun split_units(int first, int len, int unit, int split, int nsplit) {
    const int u0 = first / unit;
    const int n = (len + unit - 1) / unit - u0;
    return {u0 + (int)((long long)n * split / nsplit), u0 + (int)((long long)n * (split + 1) / nsplit)};
}

// Element offset of slot 0 of the (page, kv head g) tile; slot s adds s * D.
__host__ __device__ __forceinline__ size_t pool_tile(int page, int g, int Hkv, int ps_log2, int D) {
    return (((size_t)page * Hkv + g) << ps_log2) * (size_t)D;
}

}  // namespace attn
