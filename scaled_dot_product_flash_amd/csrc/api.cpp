// C ABI of libattn.so: argument validation, dispatch, decode workspace.
// Every argument is checked on the host before the first HIP call, so each
// error code is reachable without a GPU.

#include "attn.h"
#include "launch.h"

#include <cmath>
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

namespace attn {

bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("ATTN_LOG");
        return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
    }();
    return on;
}

void log_dispatch(const char* fmt, ...) {
    static std::mutex m;
    char line[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(line, sizeof line, fmt, ap);
    va_end(ap);
    std::lock_guard<std::mutex> lock(m);
    std::fprintf(stderr, "[attn] %s\n", line);
}

}  // namespace attn

namespace {

// largest Sq (query rows per head) any call accepts
constexpr int kMaxRows = 1 << 30;

// A dispatch holds at most 2^32 work-items per dimension. The bf16 prefill
// kernels launch one workgroup per 128 (256 threads) or 256 (512 threads)
// query rows, the float32 one per 16 rows (256 threads), up to twice as many
// after the XCD deal rounds the grid up: at most 2^31 work-items below these
// limits.
bool prefill_grid_fits(int B, int Hq, int Sq, bool f32) {
    const long long rows_per_tile = f32 ? 16 : 128;
    const long long tiles = (long long)B * Hq * (((long long)Sq + rows_per_tile - 1) / rows_per_tile);
    return tiles <= (f32 ? (1LL << 23) : (1LL << 22));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// a*b*c*d fits in int64 (all factors >= 0)
bool product_fits(long long a, long long b, long long c, long long d) {
    const unsigned __int128 p = (unsigned __int128)a * b * c * d;
    return p < ((unsigned __int128)1 << 62);
}

int validate_prefill(const void* q, const void* k, const void* v, const void* o, int B, int Hq, int Hkv,
                     int Sq, int Sk, int D, float scale, int causal, int window, bool f32, bool* empty) {
    *empty = false;
    if (B < 0 || Sq < 0) return ATTN_ERR_SHAPE;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
    if (D != 64 && D != 128) return ATTN_ERR_HEADDIM;
    if (causal != 0 && causal != 1) return ATTN_ERR_MASK;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_MASK;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (B == 0 || Sq == 0) {
        *empty = true;
        return ATTN_OK;
    }
    if (Sk < 1) return ATTN_ERR_SHAPE;
    if (causal && Sq > Sk) return ATTN_ERR_SHAPE;
    // row counts stay far from int overflow in the launchers' tile arithmetic
    if (Sq > kMaxRows) return ATTN_ERR_SHAPE;
    if (!product_fits(B, Hq, Sq, D) || !product_fits(B, Hkv, Sk, D)) return ATTN_ERR_SHAPE;
    // one (batch, kv head) slice of K or V is addressed with 32-bit byte offsets
    if ((long long)Sk * D * 4 > 0x7FFFFFFFLL) return ATTN_ERR_SHAPE;
    // grid of either kernel (at most one workgroup per 64 rows, rounded to 8)
    if (!prefill_grid_fits(B, Hq, Sq, f32)) return ATTN_ERR_SHAPE;
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// ---- workspace of the decode and backward calls ----------------------------
// One buffer per (device, stream), grown on demand. A buffer that a larger
// request replaces is retired, not freed: kernels already enqueued on the
// stream, and HIP graphs that captured a call, keep using it, so it stays
// allocated until attn_release. The mutex is held from the size check until
// the call's kernels are enqueued, so no other host thread can replace the
// buffer in between.

struct Workspace {
    float* ptr = nullptr;
    size_t floats = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_retired;   // (device, buffer) freed by attn_release
std::map<int, int> g_cu_count;

// Caller holds g_ws_mutex.
int get_workspace(int device, hipStream_t stream, size_t floats, float** out) {
    Workspace& w = g_ws[{device, stream}];
    if (w.floats < floats) {
        // growing under stream capture would leave the graph with a buffer
        // that the next eager growth could replace; the caller must size the
        // workspace with an eager call first
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return ATTN_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return ATTN_ERR_CAPTURE;
        void* p = nullptr;
        if (hipMalloc(&p, floats * sizeof(float)) != hipSuccess || !p) return ATTN_ERR_NOMEM;
        if (w.ptr) g_retired.emplace_back(device, w.ptr);
        w.ptr = static_cast<float*>(p);
        w.floats = floats;
    }
    *out = w.ptr;
    return ATTN_OK;
}

int cu_count(int device, int* out) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_cu_count.find(device);
    if (it == g_cu_count.end()) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
            return ATTN_ERR_HIP;
        it = g_cu_count.emplace(device, n).first;
    }
    *out = it->second;
    return ATTN_OK;
}

int prefill_call(bool f32, const void* q, const void* k, const void* v, void* o, float* lse, bool want_lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int causal, int window,
                 hipStream_t stream) {
    bool empty = false;
    const int rc = validate_prefill(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, f32, &empty);
    if (rc != ATTN_OK || empty) return rc;
    if (want_lse && !lse) return ATTN_ERR_NULL;
    if (want_lse && !aligned4(lse)) return ATTN_ERR_ALIGN;
    attn::PrefillArgs a{q, k, v, o, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, want_lse ? lse : nullptr};
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return ATTN_ERR_HIP;
    const int crc = cu_count(device, &a.num_cu);
    if (crc != ATTN_OK) return crc;
    return hip_status(f32 ? attn::launch_prefill_f32(a, stream) : attn::launch_prefill_bf16(a, stream));
}

int decode_validate(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                    const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int page_size, float scale, int window,
                    const void* o) {
    if (B < 0) return ATTN_ERR_SHAPE;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
    if (D != 64 && D != 128) return ATTN_ERR_HEADDIM;
    if (page_size < 8 || page_size > 256 || (page_size & (page_size - 1)) != 0) return ATTN_ERR_PAGE;
    if (window < 0) return ATTN_ERR_MASK;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (B == 0) return ATTN_OK;
    // grid dimensions: B and the head groups index workgroups in y and z, and
    // the merge runs one workgroup per (sequence, query head)
    if (B > 65535 || Hq > 65535 || (long long)B * Hq > (1LL << 24)) return ATTN_ERR_SHAPE;
    if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !o) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) || !aligned4(page_table) ||
        !aligned4(seq_lens))
        return ATTN_ERR_ALIGN;
    return ATTN_OK;
}

int decode_call(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int page_size, float scale, int window,
                void* o, hipStream_t stream) {
    int rc = decode_validate(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, page_size, scale, window, o);
    if (rc != ATTN_OK || B == 0) return rc;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return ATTN_ERR_HIP;
    int ncu = 0;
    rc = cu_count(device, &ncu);
    if (rc != ATTN_OK) return rc;
    const bool mfma = attn::decode_on_mfma(B, Hq, Hkv, D, ncu);
    const int nsplit = attn::decode_nsplit(B, Hq, Hkv, ncu, mfma);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    float* ws = nullptr;
    rc = get_workspace(device, stream, attn::decode_workspace_floats(B, Hq, D, nsplit), &ws);
    if (rc != ATTN_OK) return rc;
    attn::DecodeArgs a{q, k_pool, v_pool, page_table, seq_lens, o, B, Hq, Hkv, D, page_size, scale, window,
                       nsplit, ws, mfma};
    return hip_status(attn::launch_decode_paged(a, stream));
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq, int Sk,
             int D, float scale, int causal, int window, hipStream_t stream) {
    return prefill_call(false, q, k, v, o, nullptr, false, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, stream);
}

int attn_fwd_f32(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq,
                 int Sk, int D, float scale, int causal, int window, hipStream_t stream) {
    return prefill_call(true, q, k, v, o, nullptr, false, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, stream);
}

int attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                 int Sq, int Sk, int D, float scale, int causal, int window, hipStream_t stream) {
    return prefill_call(false, q, k, v, o, lse, true, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, stream);
}

int attn_fwd_f32_lse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Sq, int Sk, int D, float scale, int causal, int window, hipStream_t stream) {
    return prefill_call(true, q, k, v, o, lse, true, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, stream);
}

int attn_fwd_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                   const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int D,
                   int page_size, float scale, int causal, int window, hipStream_t stream) {
    if (B < 0 || Sq < 0) return ATTN_ERR_SHAPE;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
    if (D != 64 && D != 128) return ATTN_ERR_HEADDIM;
    if (page_size < 8 || page_size > 256 || (page_size & (page_size - 1)) != 0) return ATTN_ERR_PAGE;
    if (causal != 0 && causal != 1) return ATTN_ERR_MASK;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_MASK;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (B == 0 || Sq == 0) return ATTN_OK;
    if (Sq > kMaxRows || !product_fits(B, Hq, Sq, D)) return ATTN_ERR_SHAPE;
    if (!prefill_grid_fits(B, Hq, Sq, false)) return ATTN_ERR_SHAPE;
    if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !o) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) || !aligned4(page_table) ||
        !aligned4(seq_lens) || (lse && !aligned4(lse)))
        return ATTN_ERR_ALIGN;
    attn::PrefillArgs a{q, k_pool, v_pool, o, B, Hq, Hkv, Sq, 0, D, scale, causal, window, lse,
                        page_table, seq_lens, page_size};
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return ATTN_ERR_HIP;
    const int crc = cu_count(device, &a.num_cu);
    if (crc != ATTN_OK) return crc;
    return hip_status(attn::launch_prefill_bf16(a, stream));
}

int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                      const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int page_size, float scale,
                      void* o, hipStream_t stream) {
    return decode_call(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, page_size, scale, 0, o, stream);
}

int attn_decode_paged_window(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                             const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int page_size, float scale,
                             int window, void* o, hipStream_t stream) {
    return decode_call(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, page_size, scale, window, o,
                       stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool, const int32_t* page_table,
                              const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int page_size, float scale,
                              void* o, hipStream_t stream) {
    int rc = decode_validate(q, k_pool, v_pool, page_table, seq_lens, B, Hq, Hkv, D, page_size, scale, 0, o);
    if (rc != ATTN_OK || B == 0) return rc;
    // one split per (sequence, query head) at least must fit the scratch
    const size_t per_split = (size_t)B * Hq * (size_t)(D + 2);
    if (per_split > attn::kNoallocScratchFloats) return ATTN_ERR_SCRATCH;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return ATTN_ERR_HIP;
    float* ws = nullptr;
    int ncu = 0;
    if (attn::noalloc_scratch(device, &ws, &ncu) != hipSuccess) return ATTN_ERR_HIP;
    const bool mfma = attn::decode_on_mfma(B, Hq, Hkv, D, ncu);
    int nsplit = attn::decode_nsplit(B, Hq, Hkv, ncu, mfma);
    // as many splits as the scratch holds (usually all the plain call takes)
    const int fit = (int)std::min<size_t>(64, attn::kNoallocScratchFloats / per_split);
    if (nsplit > fit) nsplit = fit;
    attn::DecodeArgs a{q, k_pool, v_pool, page_table, seq_lens, o, B, Hq, Hkv, D, page_size, scale, 0,
                       nsplit, ws, mfma};
    return hip_status(attn::launch_decode_paged(a, stream));
}

int attn_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool, const int32_t* page_table,
                   const int32_t* seq_lens, int B, int Hkv, int D, int page_size, hipStream_t stream) {
    if (B < 0) return ATTN_ERR_SHAPE;
    if (Hkv < 1) return ATTN_ERR_HEADS;
    if (D != 64 && D != 128) return ATTN_ERR_HEADDIM;
    if (page_size < 8 || page_size > 256 || (page_size & (page_size - 1)) != 0) return ATTN_ERR_PAGE;
    if (B == 0) return ATTN_OK;
    // one workgroup of 128 threads per sequence
    if (B > (1 << 24)) return ATTN_ERR_SHAPE;
    if (!k_new || !v_new || !k_pool || !v_pool || !page_table || !seq_lens) return ATTN_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
        !aligned4(page_table) || !aligned4(seq_lens))
        return ATTN_ERR_ALIGN;
    attn::AppendArgs a{k_new, v_new, k_pool, v_pool, page_table, seq_lens, B, Hkv, D, page_size};
    return hip_status(attn::launch_kv_append(a, stream));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int causal,
             int window, hipStream_t stream) {
    if (B < 0 || Sq < 0 || Sk < 0) return ATTN_ERR_SHAPE;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
    if (D != 64 && D != 128) return ATTN_ERR_HEADDIM;
    if (causal != 0 && causal != 1) return ATTN_ERR_MASK;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_MASK;
    if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
    if (B == 0 || (Sq == 0 && Sk == 0)) return ATTN_OK;
    if (Sk < 1) return ATTN_ERR_SHAPE;
    if (causal && Sq > Sk) return ATTN_ERR_SHAPE;
    // row counts stay far from int overflow in the launchers' tile arithmetic
    if (Sq > kMaxRows) return ATTN_ERR_SHAPE;
    if (!product_fits(B, Hq, Sq, D) || !product_fits(B, Hkv, Sk, D)) return ATTN_ERR_SHAPE;
    // one head's Q/dO or K/V rows (plus a tile of overrun) are addressed with
    // 32-bit byte offsets
    if ((long long)Sk * D * 4 > 0x7FFFFFFFLL || (long long)Sq * D * 4 > 0x7FFFFFFFLL) return ATTN_ERR_SHAPE;
    // grids: dQ one 256-thread workgroup per 128 query rows, dK/dV one
    // 512-thread workgroup per 256 keys (up to 16 runs each when the blocks
    // are few), both below 2^31 work-items within these limits
    if ((long long)B * Hq * (((long long)Sq + 127) / 128) > (1LL << 22) ||
        (long long)B * Hkv * (((long long)Sk + 255) / 256) > (1LL << 22))
        return ATTN_ERR_SHAPE;
    // with no query rows only dk and dv (zeros) are written; the query-side
    // tensors are empty and their pointers may be NULL
    const bool rows = Sq > 0;
    if (!dk || !dv || (rows && (!q || !k || !v || !o || !dout || !lse || !dq))) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned4(lse) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return ATTN_ERR_ALIGN;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return ATTN_ERR_HIP;
    int ncu = 0;
    const int crc = cu_count(device, &ncu);
    if (crc != ATTN_OK) return crc;
    const int kv_splits = attn::backward_kv_splits(B, Hkv, Sq, Sk, ncu);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    float* ws = nullptr;
    if (Sq > 0) {
        const size_t floats = (attn::backward_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kv_splits) + 3) / 4;
        const int rc = get_workspace(device, stream, floats, &ws);
        if (rc != ATTN_OK) return rc;
    }
    attn::BackwardArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, ws};
    a.num_cu = ncu;
    a.kv_splits = kv_splits;
    return hip_status(attn::launch_backward(a, stream));
}

const char* attn_strerror(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "invalid size (negative, zero where >= 1 is required, causal with Sq > Sk, or too large)";
        case ATTN_ERR_HEADS: return "invalid head counts (need Hq >= 1, Hkv >= 1, Hq % Hkv == 0)";
        case ATTN_ERR_HEADDIM: return "unsupported head dimension (D must be 64 or 128)";
        case ATTN_ERR_MASK: return "invalid mask arguments (causal must be 0/1; window >= 0, and for prefill only with causal)";
        case ATTN_ERR_SCALE: return "scale is not finite";
        case ATTN_ERR_PAGE: return "page_size must be a power of two in [8, 256]";
        case ATTN_ERR_ALIGN: return "a tensor pointer is not sufficiently aligned (16 bytes; 4 for int32 tables)";
        case ATTN_ERR_NOMEM: return "device memory for the library workspace could not be allocated";
        case ATTN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        case ATTN_ERR_FULL: return "the page pool has too few free pages";
        case ATTN_ERR_SEQ: return "the page pool holds no sequence with this id";
        case ATTN_ERR_CAPTURE: return "the workspace would have to grow while the stream is being captured";
        case ATTN_ERR_SCRATCH: return "the call needs more than the 16 MiB of scratch the allocation-free decode holds (B * Hq * (D + 2) * 4 bytes)";
        default: return "unknown attn status code";
    }
}

void attn_release(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (g_ws.empty() && g_retired.empty()) return;
    int prev = -1;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    for (auto& kv : g_ws)
        if (kv.second.ptr) g_retired.emplace_back(kv.first.first, kv.second.ptr);
    for (auto& r : g_retired) {
        if (hipSetDevice(r.first) == hipSuccess) {
            (void)hipDeviceSynchronize();
            (void)hipFree(r.second);
        }
    }
    g_ws.clear();
    g_retired.clear();
    if (have_prev) (void)hipSetDevice(prev);
}

}  // extern "C"
