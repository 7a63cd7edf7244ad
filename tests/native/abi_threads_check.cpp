// Concurrent host calls of the C ABI, for the thread sanitizer, against the
// stand-in HIP runtime of hip_host_stub.cpp (launches are checked and
// counted, not run). The header lets every entry point be called from
// several host threads and one page pool be shared by threads; here eight
// threads, two per stream on four streams, loop over the calls that take
// the per-(device, stream) workspace (decode, backward) with sizes that make
// it grow, the prefill and KV-append calls that take none, the
// allocation-free decode, and one shared page pool. Every call must succeed;
// the thread sanitizer reports any unsynchronised access in the library's
// host code. Exits non-zero on a failed call.

#include "attn.h"

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

extern "C" long long stub_launches();
extern "C" void stub_release();

namespace {

// never dereferenced: the stand-in runtime runs no kernel
void* const A = reinterpret_cast<void*>(0x100000);
const int32_t* const AI = reinterpret_cast<const int32_t*>(0x100000);
float* const AF = reinterpret_cast<float*>(0x100000);

std::atomic<int> g_fail{0};

void expect(int rc, int want, const char* what, int t, int i) {
    if (rc != want && g_fail.fetch_add(1) < 20)
        std::printf("FAIL thread %d iteration %d: %s returned %d, want %d\n", t, i, what, rc, want);
}

void worker(int t, int iters, attn_page_pool* pool) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(0x1000 + 0x10 * (t % 4));
    const float sc = 0.1f;
    for (int i = 0; i < iters; ++i) {
        // workspace users, with sizes that keep growing
        const int B = 1 + (7 * i + t) % 64;
        const int D = (i + t) % 2 ? 128 : 64;
        expect(attn_decode_paged(A, A, A, AI, AI, B, 32, 8, D, 16, sc, A, stream), ATTN_OK, "decode", t, i);
        expect(attn_decode_paged(A, A, A, AI, AI, B, 16, 1, D, 32, sc, A, stream), ATTN_OK, "decode mfma", t, i);
        expect(attn_decode_paged_window(A, A, A, AI, AI, B, 8, 8, D, 16, sc, 100, A, stream), ATTN_OK,
               "decode window", t, i);
        expect(attn_bwd(A, A, A, A, A, AF, A, A, A, 1, 4, 2, 64 + 32 * (i % 9), 64 + 32 * (i % 9), D, sc, 1, 0,
                        stream),
               ATTN_OK, "backward", t, i);
        expect(attn_bwd(A, A, A, A, A, AF, A, A, A, 1, 8, 1, 100, 3000, 128, sc, 1, 0, stream), ATTN_OK,
               "backward split", t, i);
        // no workspace
        expect(attn_fwd(A, A, A, A, 2, 8, 2, 100 + i, 300, D, sc, 1, 0, stream), ATTN_OK, "prefill", t, i);
        expect(attn_fwd_paged(A, A, A, AI, AI, A, AF, 3, 8, 2, 64, D, 16, sc, 1, 0, stream), ATTN_OK,
               "paged prefill", t, i);
        expect(attn_kv_append(A, A, A, A, AI, AI, B, 2, D, 16, stream), ATTN_OK, "kv append", t, i);
        expect(attn_decode_paged_noalloc(A, A, A, AI, AI, 4, 8, 2, D, 16, sc, A, stream), ATTN_OK, "noalloc", t,
               i);
        // the shared page pool: this thread's sequences only
        const int64_t ids[2] = {1000 * t + 1, 1000 * t + 2};
        expect(attn_pages_resize(pool, ids[0], 1 + (i * 13) % 200), ATTN_OK, "pages resize", t, i);
        expect(attn_pages_resize(pool, ids[1], (i * 29) % 300), ATTN_OK, "pages resize", t, i);
        int32_t table[64], lens[2];
        int64_t n = 0;
        const int rc = attn_pages_table(pool, ids, (i * 29) % 300 ? 2 : 1, table, 64, lens, &n);
        expect(rc, ATTN_OK, "pages table", t, i);
        if (attn_pages_free_count(pool) < 0) expect(-1, 0, "free count", t, i);
    }
}

}  // namespace

int main(int argc, char** argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 200;
    attn_page_pool* pool = nullptr;
    if (attn_pages_create(8 * 64, 16, &pool) != ATTN_OK) {
        std::printf("FAIL pool\n");
        return 1;
    }
    std::vector<std::thread> threads;
    for (int t = 0; t < 8; ++t) threads.emplace_back(worker, t, iters, pool);
    for (auto& th : threads) th.join();
    attn_pages_destroy(pool);
    attn_release();
    stub_release();
    if (g_fail.load()) {
        std::printf("%d failed calls\n", g_fail.load());
        return 1;
    }
    std::printf("thread checks ok, launches %lld\n", stub_launches());
    return 0;
}
