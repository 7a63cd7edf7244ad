// Host replay of the paged-cache accesses of the decode, paged prefill and KV
// append kernels: the loops over blocks, tiles, DMA slots and lanes that the
// kernels run, with the index arithmetic of paging.h that they call. For
// random ragged caches (page sizes 8-256, lengths 1-20000, windows, context
// splits 1-64) every page-table read must fall in the sequence's own entries,
// every element read in the pool, every row in the page of its token, and the
// decode loops must visit each visible token exactly once (K and V alike).
// Prints one line per family and exits non-zero on the first failure.

#include "paging.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <vector>

namespace {

struct Cache {
    int ps_log2, Hkv, D;
    std::vector<int> lens, off, table;
    long long pool_elems() const { return (long long)table.size() * Hkv * (1 << ps_log2) * D; }
};

Cache make_cache(std::mt19937& rng, int B, int ps_log2, int Hkv, int D, int len_hi) {
    Cache c{ps_log2, Hkv, D, {}, {}, {}};
    int total = 0;
    for (int b = 0; b < B; ++b) {
        int len = 1 + (int)(rng() % len_hi);
        if (rng() % 5 == 0) len = 1 + (int)(rng() % 3);                  // tiny
        if (rng() % 7 == 0) len = (1 << ps_log2) * (1 + (int)(rng() % 4)); // page multiples
        c.lens.push_back(len);
        c.off.push_back(total);
        total += attn::seq_pages(len, ps_log2);
    }
    c.table.resize(total);
    std::iota(c.table.begin(), c.table.end(), 0);
    std::shuffle(c.table.begin(), c.table.end(), rng);
    return c;
}

int g_fail = 0;
#define CHECK(cond, ...)                                     \
    do {                                                     \
        if (!(cond)) {                                       \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
            std::printf(__VA_ARGS__);                        \
            std::printf("\n");                               \
            if (++g_fail > 10) std::exit(1);                 \
        }                                                    \
    } while (0)

// a page-table read of sequence b at the entry holding token t
int read_entry(const Cache& c, int b, int entry) {
    const int n = attn::seq_pages(c.lens[b], c.ps_log2);
    CHECK(entry >= c.off[b] && entry < c.off[b] + n, "table entry %d outside sequence %d's [%d, %d)", entry, b,
          c.off[b], c.off[b] + n);
    return c.table[std::min(std::max(entry, 0), (int)c.table.size() - 1)];
}

// an element read of `count` elements at `elem`, which must be token t's row
// of kv head g (columns col .. col + count - 1)
void read_row(const Cache& c, long long elem, int count, int b, int t, int g, int col) {
    CHECK(elem >= 0 && elem + count <= c.pool_elems(), "element %lld outside the pool", elem);
    const int ps = 1 << c.ps_log2;
    // the layout's definition, written out independently of paging.h
    const long long want = (((long long)c.table[c.off[b] + t / ps] * c.Hkv + g) * ps + t % ps) * c.D + col;
    CHECK(elem == want, "sequence %d token %d head %d: element %lld, want %lld", b, t, g, elem, want);
}

// decode_split_kernel (vector ALU): per split, blocks of TB tokens, four
// loads of TPI tokens each, lane (r, c) reading 8 dims of token t0 + r
void decode_vector(const Cache& c, int window, int nsplit, int g) {
    const int CPT = c.D / 8, TPI = 64 / CPT, TB = 4 * TPI;
    for (size_t b = 0; b < c.lens.size(); ++b) {
        const int len = c.lens[b];
        const int first = attn::window_first(len, window);
        std::vector<int> seen(len, 0);
        for (int split = 0; split < nsplit; ++split) {
            const attn::UnitRun run = attn::split_units(first, len, TB, split, nsplit);
            for (int blk = run.begin; blk < run.end; ++blk)
                for (int i = 0; i < 4; ++i) {
                    const int t0 = blk * TB + i * TPI;
                    if (t0 >= len) continue;
                    const int page = read_entry(c, (int)b, c.off[b] + (t0 >> c.ps_log2));
                    const size_t tile = attn::pool_tile(page, g, c.Hkv, c.ps_log2, c.D) +
                                        (size_t)(t0 & ((1 << c.ps_log2) - 1)) * c.D;
                    for (int r = 0; r < TPI; ++r) {
                        const int t = t0 + r;
                        // tokens past the length sit in the same page (read,
                        // then excluded by selection): the row must still be
                        // that slot of this page
                        CHECK((t0 & ((1 << c.ps_log2) - 1)) + r < (1 << c.ps_log2), "load crosses a page");
                        if (t < len) {
                            for (int col = 0; col < c.D; col += 8) read_row(c, (long long)tile + r * c.D + col, 8, (int)b, t, g, col);
                            if (t >= first) ++seen[t];
                        }
                    }
                }
        }
        for (int t = first; t < len; ++t) CHECK(seen[t] == 1, "vector decode: token %d of %d read %d times", t, len, seen[t]);
    }
}

// decode_mfma_kernel: 32-token tiles dealt to four waves; K rows into
// registers (token clamped to len - 1), V slots of RPS rows by DMA
void decode_mfma(const Cache& c, int window, int nsplit, int g) {
    const int kTT = 32, CPR = c.D / 8, RPS = 64 / CPR, VSLOTS = kTT * c.D * 2 / 1024;
    const int ps = 1 << c.ps_log2;
    for (size_t b = 0; b < c.lens.size(); ++b) {
        const int len = c.lens[b];
        const int first = attn::window_first(len, window);
        const int last_page = (len - 1) >> c.ps_log2;
        std::vector<int> seen_k(len, 0), seen_v(len, 0);
        for (int split = 0; split < nsplit; ++split) {
            const attn::UnitRun run = attn::split_units(first, len, kTT, split, nsplit);
            for (int wave = 0; wave < 4; ++wave)
                for (int t = run.begin + wave; t < run.end; t += 4) {
                    const int j0 = t * kTT, p0 = j0 >> c.ps_log2;
                    int pid[4];
                    for (int i = 0; i < 4; ++i) pid[i] = read_entry(c, (int)b, c.off[b] + std::min(p0 + i, last_page));
                    for (int ln = 0; ln < 32; ++ln) {
                        const int tok = std::min(j0 + ln, len - 1);
                        const int idx = (tok >> c.ps_log2) - p0;
                        CHECK(idx >= 0 && idx <= 3, "K token %d needs page %d of the tile's four", tok, idx);
                        const size_t kp = attn::pool_tile(pid[std::min(std::max(idx, 0), 3)], g, c.Hkv, c.ps_log2, c.D) +
                                          (size_t)(tok & (ps - 1)) * c.D;
                        for (int col = 0; col < c.D; col += 8) read_row(c, (long long)kp + col, 8, (int)b, tok, g, col);
                        if (j0 + ln < len && j0 + ln >= first) ++seen_k[j0 + ln];
                    }
                    for (int sl = 0; sl < VSLOTS; ++sl) {
                        const int r0 = j0 + sl * RPS;
                        if (r0 >= len) continue;   // zero-size range: no read
                        const int idx = (r0 >> c.ps_log2) - p0;
                        CHECK(idx >= 0 && idx <= 3, "V slot row %d needs page %d of the tile's four", r0, idx);
                        const size_t tile = attn::pool_tile(pid[std::min(std::max(idx, 0), 3)], g, c.Hkv, c.ps_log2, c.D);
                        for (int rr = 0; rr < RPS; ++rr) {
                            const int j = r0 + rr;
                            if (j >= len) continue;   // offset past the range: reads zeros
                            CHECK((j >> c.ps_log2) == (r0 >> c.ps_log2), "V slot crosses a page");
                            const long long off = (long long)(j & (ps - 1)) * c.D;
                            CHECK(off + c.D <= (long long)ps * c.D, "V row beyond the buffer range");
                            for (int col = 0; col < c.D; col += 8) read_row(c, (long long)tile + off + col, 8, (int)b, j, g, col);
                            if (j >= first) ++seen_v[j];
                        }
                    }
                }
        }
        for (int t = first; t < len; ++t) {
            CHECK(seen_k[t] == 1, "mfma decode: K token %d of %d read %d times", t, len, seen_k[t]);
            CHECK(seen_v[t] == 1, "mfma decode: V token %d of %d read %d times", t, len, seen_v[t]);
        }
    }
}

// paged prefill: every 64-key tile of the sequence, DMA slots of `rows`
// consecutive rows (4 for the D = 128 kernels with NW waves, 8 for D = 64
// with four waves); a slot wholly past the length reads nothing, rows past it
// read zeros
void prefill_paged(const Cache& c, int NW, int g) {
    const int BN = 64, ps = 1 << c.ps_log2;
    const int rows = c.D == 128 ? 4 : 8;
    const int slots = BN * c.D * 2 / 1024;
    for (size_t b = 0; b < c.lens.size(); ++b) {
        const int Sk = c.lens[b];
        for (int t = 0; t * BN < Sk; ++t)
            for (int sl = 0; sl < slots; ++sl) {
                // the D = 128 kernels give slot wave + NW i the rows
                // t * BN + 4 NW i + 4 wave; the D = 64 kernel slot sl the rows
                // t * BN + 8 sl: both are t * BN + rows * sl
                const int j0 = t * BN + rows * sl;
                if (j0 >= Sk) continue;
                const int page = read_entry(c, (int)b, c.off[b] + (j0 >> c.ps_log2));
                const size_t tile = attn::pool_tile(page, g, c.Hkv, c.ps_log2, c.D);
                for (int r = 0; r < rows; ++r) {
                    const int j = j0 + r;
                    if (j >= Sk) continue;
                    CHECK((j >> c.ps_log2) == (j0 >> c.ps_log2), "prefill slot crosses a page");
                    for (int col = 0; col < c.D; col += 8)
                        read_row(c, (long long)tile + (long long)(j & (ps - 1)) * c.D + col, 8, (int)b, j, g, col);
                }
            }
        (void)NW;
    }
}

// kv_append: the new token at position len - 1
void kv_append(const Cache& c) {
    const int ps = 1 << c.ps_log2;
    for (size_t b = 0; b < c.lens.size(); ++b) {
        const int t = c.lens[b] - 1;
        const int page = read_entry(c, (int)b, c.off[b] + (t >> c.ps_log2));
        for (int g = 0; g < c.Hkv; ++g) {
            const size_t dst = attn::pool_tile(page, 0, c.Hkv, c.ps_log2, c.D) + (size_t)(t & (ps - 1)) * c.D +
                               (size_t)g * ps * c.D;
            for (int col = 0; col < c.D; col += 8) read_row(c, (long long)dst + col, 8, (int)b, t, g, col);
        }
    }
}

}  // namespace

int main() {
    std::mt19937 rng(2024);
    int cases = 0;
    for (int it = 0; it < 300; ++it) {
        const int ps_log2 = 3 + (int)(rng() % 6);
        const int D = rng() % 2 ? 128 : 64;
        const int Hkv = 1 + (int)(rng() % 4);
        const int B = 1 + (int)(rng() % 12);
        const int len_hi = it % 10 == 0 ? 20000 : 1 + (int)(rng() % 3000);
        const Cache c = make_cache(rng, B, ps_log2, Hkv, D, len_hi);
        const int windows[] = {0, 1, 7, 100, 4096, 1 << 30};
        const int window = windows[rng() % 6];
        const int nsplit = 1 + (int)(rng() % 64);
        const int g = (int)(rng() % Hkv);
        decode_vector(c, window, nsplit, g);
        decode_mfma(c, window, nsplit, g);
        prefill_paged(c, rng() % 2 ? 8 : 4, g);
        kv_append(c);
        ++cases;
    }
    if (g_fail) {
        std::printf("%d failures\n", g_fail);
        return 1;
    }
    std::printf("decode (vector, mfma), paged prefill, kv append: %d random caches ok\n", cases);
    return 0;
}
