// Host code of the C ABI under the address and undefined-behaviour
// sanitizers, against the stand-in HIP runtime of hip_host_stub.cpp (one
// device of 256 CUs; launches are checked against the hardware's limits and
// counted, not run). Three parts:
//  1. argument validation: each documented error code of each entry point;
//  2. a sweep of every entry point over boundary values of every size and
//     mask argument (several hundred thousand calls): each call must return a
//     documented code, a call that returns ATTN_OK must have launched kernels
//     (or be an empty call), and the sanitizers must stay silent;
//  3. the page pool under random resizes, checked against a model.
// Exits non-zero (or aborts with a sanitizer report) on the first failure.

#include "attn.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <map>
#include <random>
#include <set>
#include <vector>

extern "C" long long stub_launches();
extern "C" void stub_set_capturing(int on);
extern "C" void stub_set_no_device(int on);
extern "C" void stub_release();

namespace {

int g_fail = 0;
#define CHECK(cond, ...)                                         \
    do {                                                         \
        if (!(cond)) {                                           \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);     \
            std::printf(__VA_ARGS__);                            \
            std::printf("\n");                                   \
            if (++g_fail > 20) std::exit(1);                     \
        }                                                        \
    } while (0)

// never dereferenced: the stand-in runtime runs no kernel
void* const A = reinterpret_cast<void*>(0x100000);
void* const U = reinterpret_cast<void*>(0x100002);
const int32_t* const AI = reinterpret_cast<const int32_t*>(0x100000);
const float NaN = std::numeric_limits<float>::quiet_NaN();
const float Inf = std::numeric_limits<float>::infinity();

bool documented(int rc) { return rc <= 0 && rc >= ATTN_ERR_SCRATCH; }

void validation() {
    // prefill (every variant validates the shared arguments the same way)
    auto fwd = [](int B, int Hq, int Hkv, int Sq, int Sk, int D, float sc, int causal, int window, void* q = A) {
        const int r0 = attn_fwd(q, A, A, A, B, Hq, Hkv, Sq, Sk, D, sc, causal, window, nullptr);
        const int r1 = attn_fwd_f32(q, A, A, A, B, Hq, Hkv, Sq, Sk, D, sc, causal, window, nullptr);
        const int r2 = attn_fwd_lse(q, A, A, A, (float*)A, B, Hq, Hkv, Sq, Sk, D, sc, causal, window, nullptr);
        CHECK(r0 == r1 && r1 == r2, "prefill variants disagree: %d %d %d", r0, r1, r2);
        return r0;
    };
    CHECK(fwd(1, 4, 2, 8, 8, 64, 0.1f, 1, 0, nullptr) == ATTN_ERR_NULL, "null q");
    CHECK(fwd(-1, 4, 2, 8, 8, 64, 0.1f, 1, 0) == ATTN_ERR_SHAPE, "B < 0");
    CHECK(fwd(1, 4, 2, 9, 8, 64, 0.1f, 1, 0) == ATTN_ERR_SHAPE, "causal Sq > Sk");
    CHECK(fwd(1, 6, 4, 8, 8, 64, 0.1f, 1, 0) == ATTN_ERR_HEADS, "Hq % Hkv");
    CHECK(fwd(1, 4, 2, 8, 8, 96, 0.1f, 1, 0) == ATTN_ERR_HEADDIM, "D 96");
    CHECK(fwd(1, 4, 2, 8, 8, 64, 0.1f, 0, 3) == ATTN_ERR_MASK, "window without causal");
    CHECK(fwd(1, 4, 2, 8, 8, 64, NaN, 1, 0) == ATTN_ERR_SCALE, "NaN scale");
    CHECK(fwd(1, 4, 2, 8, 8, 64, 0.1f, 1, 0, U) == ATTN_ERR_ALIGN, "misaligned q");
    CHECK(fwd(1, 4, 2, 8, 8, 64, 0.1f, 1, 0) == ATTN_OK, "valid prefill");
    // decode (plain, windowed, allocation-free)
    auto dec = [](int B, int Hq, int Hkv, int D, int ps, float sc, void* q = A) {
        const int r0 = attn_decode_paged(q, A, A, AI, AI, B, Hq, Hkv, D, ps, sc, A, nullptr);
        const int r1 = attn_decode_paged_window(q, A, A, AI, AI, B, Hq, Hkv, D, ps, sc, 5, A, nullptr);
        const int r2 = attn_decode_paged_noalloc(q, A, A, AI, AI, B, Hq, Hkv, D, ps, sc, A, nullptr);
        CHECK(r0 == r1, "decode variants disagree: %d %d", r0, r1);
        CHECK(r0 == r2 || r2 == ATTN_ERR_SCRATCH, "noalloc disagrees: %d %d", r0, r2);
        return r0;
    };
    CHECK(dec(2, 8, 2, 128, 16, 0.1f, nullptr) == ATTN_ERR_NULL, "decode null");
    CHECK(dec(65536, 8, 2, 128, 16, 0.1f) == ATTN_ERR_SHAPE, "decode B > 65535");
    CHECK(dec(2, 8, 3, 128, 16, 0.1f) == ATTN_ERR_HEADS, "decode heads");
    CHECK(dec(2, 8, 2, 128, 12, 0.1f) == ATTN_ERR_PAGE, "decode page 12");
    CHECK(dec(2, 8, 2, 128, 16, Inf) == ATTN_ERR_SCALE, "decode inf scale");
    CHECK(dec(2, 8, 2, 128, 16, 0.1f) == ATTN_OK, "valid decode");
    CHECK(attn_decode_paged_window(A, A, A, AI, AI, 2, 8, 2, 128, 16, 0.1f, -1, A, nullptr) == ATTN_ERR_MASK,
          "negative window");
    CHECK(attn_decode_paged_noalloc(A, A, A, AI, AI, 32264, 1, 1, 128, 16, 0.1f, A, nullptr) == ATTN_ERR_SCRATCH,
          "noalloc beyond scratch");
    // workspace growth under capture
    stub_set_capturing(1);
    CHECK(attn_decode_paged(A, A, A, AI, AI, 2, 8, 2, 128, 16, 0.1f, A, nullptr) == ATTN_OK,
          "capture with a large enough workspace");
    CHECK(attn_decode_paged(A, A, A, AI, AI, 4000, 32, 8, 128, 16, 0.1f, A, nullptr) == ATTN_ERR_CAPTURE,
          "growth under capture");
    stub_set_capturing(0);
    // no device: the HIP error surfaces, nothing else
    stub_set_no_device(1);
    CHECK(fwd(1, 4, 2, 8, 8, 64, 0.1f, 1, 0) == ATTN_ERR_HIP, "no device");
    stub_set_no_device(0);
    // kv append, paged prefill, backward
    CHECK(attn_kv_append(A, A, A, A, AI, AI, 2, 2, 96, 16, nullptr) == ATTN_ERR_HEADDIM, "append D");
    CHECK(attn_kv_append(A, A, A, A, AI, AI, 2, 2, 128, 16, nullptr) == ATTN_OK, "valid append");
    CHECK(attn_fwd_paged(A, A, A, AI, AI, A, nullptr, 2, 8, 2, 16, 128, 16, 0.1f, 0, 3, nullptr) == ATTN_ERR_MASK,
          "paged window without causal");
    CHECK(attn_fwd_paged(A, A, A, AI, AI, A, nullptr, 2, 8, 2, 16, 128, 16, 0.1f, 1, 0, nullptr) == ATTN_OK,
          "valid paged prefill");
    CHECK(attn_bwd(A, A, A, A, A, (float*)A, A, A, A, 1, 4, 2, 8, 8, 128, 0.1f, 1, 0, nullptr) == ATTN_OK,
          "valid backward");
    CHECK(attn_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, A, A, 1, 4, 2, 0, 8, 128, 0.1f,
                   0, 0, nullptr) == ATTN_OK, "backward without query rows");
    for (int c = ATTN_ERR_SCRATCH; c <= 0; ++c) CHECK(attn_strerror(c) != nullptr, "strerror %d", c);
}

const int kInts[] = {std::numeric_limits<int>::min(), -1, 0, 1, 2, 3, 7, 8, 31, 32, 33, 63, 64, 65, 127, 128,
                     129, 255, 256, 257, 1000, 2048, 2049, 4096, 16384, 65535, 65536, 1 << 20, 1 << 24, 1 << 28,
                     std::numeric_limits<int>::max() - 1, std::numeric_limits<int>::max()};
const int kHeads[] = {0, 1, 2, 3, 4, 8, 12, 32, 64, 65535, 65536, std::numeric_limits<int>::max()};
const int kD[] = {0, 32, 64, 96, 128, 256};
const int kPs[] = {0, 4, 8, 12, 16, 32, 256, 512};
const float kScale[] = {0.f, 0.125f, -0.3f, 1e30f, -1e-30f};

void sweep(unsigned seed, long long calls) {
    std::mt19937 rng(seed);
    auto pick = [&](const auto& arr) { return arr[rng() % (sizeof(arr) / sizeof(arr[0]))]; };
    const int kSane[] = {1, 2, 3, 17, 64, 100, 129, 256, 1000, 4096, 5000, 16384};
    for (long long i = 0; i < calls; ++i) {
        // half the calls draw every argument from boundary values (mostly
        // invalid), half from shapes that pass validation and reach the
        // launchers
        const bool sane = rng() % 2;
        const int B = sane ? pick(kSane) % 97 + 1 : pick(kInts) % 100003;
        const int Hq = sane ? 8 * (1 + (int)(rng() % 8)) : pick(kHeads);
        const int Sq = sane ? pick(kSane) : pick(kInts);
        const int Sk = sane ? Sq + (int)(rng() % 3) * pick(kSane) : pick(kInts);
        const int D = sane ? (rng() % 2 ? 64 : 128) : pick(kD);
        int Hkv = pick(kHeads);
        if ((sane || rng() % 2) && Hq > 0) Hkv = Hq / (1 << (rng() % 4));
        const int causal = sane ? (int)(rng() % 2) : (int)(rng() % 3) == 2 ? (int)(rng() % 5) - 2 : (int)(rng() % 2);
        const int window = rng() % 3 ? 0 : sane ? pick(kSane) : pick(kInts);
        const float scale = pick(kScale);
        const int ps = sane ? 8 << (rng() % 6) : pick(kPs);
        const long long before = stub_launches();
        int rc = 0;
        bool empty = false;
        switch (rng() % 7) {
            case 0:
                rc = attn_fwd(A, A, A, A, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, nullptr);
                empty = B == 0 || Sq == 0;
                break;
            case 1:
                rc = attn_fwd_f32_lse(A, A, A, A, (float*)A, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, nullptr);
                empty = B == 0 || Sq == 0;
                break;
            case 2:
                rc = attn_fwd_paged(A, A, A, AI, AI, A, (float*)A, B, Hq, Hkv, Sq, D, ps, scale, causal, window,
                                    nullptr);
                empty = B == 0 || Sq == 0;
                break;
            case 3:
                rc = attn_decode_paged_window(A, A, A, AI, AI, B, Hq, Hkv, D, ps, scale, window, A, nullptr);
                empty = B == 0;
                break;
            case 4:
                rc = attn_decode_paged_noalloc(A, A, A, AI, AI, B, Hq, Hkv, D, ps, scale, A, nullptr);
                empty = B == 0;
                break;
            case 5:
                rc = attn_kv_append(A, A, A, A, AI, AI, B, Hkv, D, ps, nullptr);
                empty = B == 0;
                break;
            default:
                rc = attn_bwd(A, A, A, A, A, (float*)A, A, A, A, B, Hq, Hkv, Sq, Sk, D, scale, causal, window,
                              nullptr);
                empty = B == 0 || (Sq == 0 && Sk == 0);
                break;
        }
        CHECK(documented(rc), "undocumented status %d", rc);
        if (rc == ATTN_OK && !empty)
            CHECK(stub_launches() > before, "ATTN_OK without a launch: B %d Hq %d Hkv %d Sq %d Sk %d D %d", B, Hq, Hkv,
                  Sq, Sk, D);
        if (rc != ATTN_OK) CHECK(stub_launches() == before, "an error (%d) after a launch", rc);
    }
}

void page_pool(unsigned seed) {
    std::mt19937 rng(seed);
    const int ps = 16, num_pages = 96;
    attn_page_pool* pool = nullptr;
    CHECK(attn_pages_create(num_pages, ps, &pool) == ATTN_OK && pool, "create");
    std::map<int64_t, int> model;
    for (int it = 0; it < 20000; ++it) {
        const int64_t sid = (int64_t)(rng() % 16) - 3;
        const int choice = (int)(rng() % 4);
        const int cur = model.count(sid) ? model[sid] : 0;
        const int len = choice == 0 ? 0 : choice == 1 ? (int)(rng() % 40) : choice == 2 ? (int)(rng() % 600) : cur + 1;
        int owned = 0;
        for (auto& kv : model) owned += (kv.second + ps - 1) / ps;
        const int rc = attn_pages_resize(pool, sid, len);
        const int need = (len + ps - 1) / ps;
        const int have_pages = model.count(sid) ? (model[sid] + ps - 1) / ps : 0;
        if (need - have_pages > num_pages - owned) {
            CHECK(rc == ATTN_ERR_FULL, "expected FULL, got %d", rc);
        } else {
            CHECK(rc == ATTN_OK, "resize failed %d", rc);
            if (len == 0) model.erase(sid); else model[sid] = len;
        }
        if (it % 97 == 0) {
            std::vector<int64_t> ids;
            for (auto& kv : model) ids.push_back(kv.first);
            std::vector<int32_t> table(num_pages + 1), lens(ids.size() + 1);
            int64_t n = -1;
            const int trc = attn_pages_table(pool, ids.data(), (int)ids.size(), table.data(),
                                             (int64_t)table.size(), lens.data(), &n);
            CHECK(trc == ATTN_OK, "table %d", trc);
            std::set<int32_t> seen;
            int64_t expect = 0;
            for (size_t i = 0; i < ids.size(); ++i) {
                CHECK(lens[i] == model[ids[i]], "length");
                expect += (lens[i] + ps - 1) / ps;
            }
            CHECK(n == expect, "table length %lld vs %lld", (long long)n, (long long)expect);
            for (int64_t i = 0; i < n; ++i) {
                CHECK(table[i] >= 0 && table[i] < num_pages, "page id");
                CHECK(seen.insert(table[i]).second, "page owned twice");
            }
            CHECK(attn_pages_free_count(pool) == num_pages - (int)n, "free count");
        }
    }
    attn_pages_destroy(pool);
}

// one valid call of each launch shape, each of which must launch: the
// workloads of the bench and the dispatch branches (eight or four waves,
// D = 64, paged, vector or MFMA decode, backward with split reduction)
void dispatch_examples() {
    const long long before = stub_launches();
    CHECK(attn_fwd(A, A, A, A, 4, 32, 8, 4096, 4096, 128, 0.088f, 1, 0, nullptr) == ATTN_OK, "fwd c3");
    CHECK(attn_fwd(A, A, A, A, 8, 12, 12, 1024, 1024, 64, 0.125f, 1, 0, nullptr) == ATTN_OK, "fwd D=64");
    CHECK(attn_fwd(A, A, A, A, 1, 16, 16, 2048, 2048, 128, -0.088f, 1, 512, nullptr) == ATTN_OK, "fwd 4 waves");
    CHECK(attn_fwd_f32(A, A, A, A, 1, 1, 1, 128, 128, 64, 0.125f, 0, 0, nullptr) == ATTN_OK, "fwd f32");
    CHECK(attn_fwd_paged(A, A, A, AI, AI, A, nullptr, 8, 32, 8, 512, 128, 16, 0.088f, 1, 0, nullptr) == ATTN_OK,
          "fwd paged");
    CHECK(attn_decode_paged(A, A, A, AI, AI, 64, 32, 8, 128, 16, 0.088f, A, nullptr) == ATTN_OK, "decode");
    CHECK(attn_decode_paged(A, A, A, AI, AI, 8, 64, 8, 128, 16, 0.088f, A, nullptr) == ATTN_OK, "decode mfma");
    const float* const AF = reinterpret_cast<const float*>(A);
    CHECK(attn_bwd(A, A, A, A, A, AF, A, A, A, 1, 8, 2, 1024, 1024, 128, 0.088f, 1, 0, nullptr) == ATTN_OK, "bwd");
    CHECK(attn_kv_append(A, A, A, A, AI, AI, 4, 8, 128, 16, nullptr) == ATTN_OK, "append");
    CHECK(stub_launches() - before >= 12, "dispatch examples launched %lld kernels", stub_launches() - before);
}

}  // namespace

int main(int argc, char** argv) {
    const long long calls = argc > 1 ? std::atoll(argv[1]) : 200000;
    validation();
    dispatch_examples();
    for (unsigned s = 0; s < 4; ++s) sweep(s, calls / 4);
    page_pool(7);
    page_pool(8);
    attn_release();
    attn_release();
    stub_release();
    std::printf("launches %lld\n", stub_launches());
    if (g_fail) {
        std::printf("%d failures\n", g_fail);
        return 1;
    }
    std::printf("host checks ok\n");
    return 0;
}
