// Host-side page allocator for the paged KV cache.
//
// "LLM 核心技术：Attention 机制的实现与优化" (PagedAttention section) and
// "Attention From Scratch" (paged-KV-cache part) describe the cache as fixed-
// size pages taken from one global pool and handed to sequences on demand, a
// page table per sequence recording where its logical pages live, and pages
// returned to the pool when a sequence shrinks or ends. This file keeps that
// bookkeeping on the host: a free list of physical page ids and, per sequence,
// its length and its pages in logical order. attn_pages_table writes the
// ragged page table and seq_lens that attn_decode_paged, attn_kv_append and
// attn_decode_paged_window read.
//
// The free list is a stack; the pool starts with pages handed out in
// increasing order, and a freed page is the next one handed out. Every entry
// point locks the pool's mutex.

#include "attn.h"

#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

struct attn_page_pool {
    int num_pages = 0;
    int page_size = 0;
    std::vector<int32_t> free_pages;  // stack, back() is handed out next
    struct Seq {
        int len = 0;
        std::vector<int32_t> pages;   // logical order
    };
    std::unordered_map<int64_t, Seq> seqs;
    mutable std::mutex mu;
};

namespace {

bool valid_page_size(int ps) { return ps >= 8 && ps <= 256 && (ps & (ps - 1)) == 0; }

int pages_for(int len, int ps) { return (len + ps - 1) / ps; }

}  // namespace

extern "C" {

int attn_pages_create(int num_pages, int page_size, attn_page_pool** out) {
    if (!out) return ATTN_ERR_NULL;
    *out = nullptr;
    if (num_pages < 1) return ATTN_ERR_SHAPE;
    if (!valid_page_size(page_size)) return ATTN_ERR_PAGE;
    attn_page_pool* p = new (std::nothrow) attn_page_pool;
    if (!p) return ATTN_ERR_NOMEM;
    try {
        p->free_pages.resize(num_pages);
    } catch (...) {
        delete p;
        return ATTN_ERR_NOMEM;
    }
    for (int i = 0; i < num_pages; ++i) p->free_pages[i] = num_pages - 1 - i;
    p->num_pages = num_pages;
    p->page_size = page_size;
    *out = p;
    return ATTN_OK;
}

void attn_pages_destroy(attn_page_pool* pool) { delete pool; }

int attn_pages_resize(attn_page_pool* pool, int64_t seq_id, int len) {
    if (!pool) return ATTN_ERR_NULL;
    if (len < 0) return ATTN_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(pool->mu);
    auto it = pool->seqs.find(seq_id);
    const int have = it == pool->seqs.end() ? 0 : (int)it->second.pages.size();
    const int need = pages_for(len, pool->page_size);
    if (need > have && need - have > (int)pool->free_pages.size()) return ATTN_ERR_FULL;
    if (len == 0) {
        if (it != pool->seqs.end()) {
            auto& pages = it->second.pages;
            for (auto r = pages.rbegin(); r != pages.rend(); ++r) pool->free_pages.push_back(*r);
            pool->seqs.erase(it);
        }
        return ATTN_OK;
    }
    try {
        attn_page_pool::Seq& s = pool->seqs[seq_id];
        s.pages.reserve(need);
        while ((int)s.pages.size() < need) {
            s.pages.push_back(pool->free_pages.back());
            pool->free_pages.pop_back();
        }
        while ((int)s.pages.size() > need) {
            pool->free_pages.push_back(s.pages.back());
            s.pages.pop_back();
        }
        s.len = len;
    } catch (...) {
        return ATTN_ERR_NOMEM;
    }
    return ATTN_OK;
}

int attn_pages_free_count(const attn_page_pool* pool) {
    if (!pool) return ATTN_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    return (int)pool->free_pages.size();
}

int attn_pages_table(const attn_page_pool* pool, const int64_t* seq_ids, int n, int32_t* page_table,
                     int64_t table_cap, int32_t* seq_lens, int64_t* table_len) {
    if (!pool || !table_len) return ATTN_ERR_NULL;
    if (n < 0 || table_cap < 0) return ATTN_ERR_SHAPE;
    *table_len = 0;
    if (n == 0) return ATTN_OK;
    if (!seq_ids || !seq_lens) return ATTN_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it == pool->seqs.end()) return ATTN_ERR_SEQ;
        total += (int64_t)it->second.pages.size();
    }
    *table_len = total;
    if (total > table_cap) return ATTN_ERR_SHAPE;
    if (total > 0 && !page_table) return ATTN_ERR_NULL;
    int64_t at = 0;
    for (int i = 0; i < n; ++i) {
        const auto& s = pool->seqs.find(seq_ids[i])->second;
        seq_lens[i] = s.len;
        std::copy(s.pages.begin(), s.pages.end(), page_table + at);
        at += (int64_t)s.pages.size();
    }
    return ATTN_OK;
}

}  // extern "C"
