// Internal interface between the C ABI (api.cpp) and the kernel files.
// Arguments arrive here already validated; nothing in this header is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace attn {

// Orders one wave's LDS accesses across lanes: every lane's accesses before
// the call come before every lane's accesses after it. The LDS executes a
// wave's instructions in order, so this only keeps the compiler, which
// reasons about one lane at a time, from moving an access across it; it
// emits no instruction. Used where lanes exchange data through LDS (write in
// one layout, read another lane's values back) and where such a region is
// written again after it was read.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ATTN_LOG=1 in the environment (read once per process): every launch
// decision (kernel, grid, work split) goes to stderr as one "[attn]" line.
bool log_enabled();
void log_dispatch(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// A dispatch holds the grid size in work-items, 32 bits per dimension.
inline bool grid_fits(long long workgroups, int threads) {
    return workgroups > 0 && workgroups * (long long)threads < (1LL << 32);
}

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int B, Hq, Hkv, Sq, Sk, D;
    float scale;
    int causal, window;
    float* lse;     // [B, Hq, Sq] float32 log-sum-exp per row, or nullptr
    // paged K/V (k, v are then [pages, Hkv, page_size, D] pools and Sk is
    // per sequence); nullptr page_table: contiguous [B, Hkv, Sk, D]
    const int32_t* page_table = nullptr;
    const int32_t* seq_lens = nullptr;
    int page_size = 0;
    int num_cu = 0;  // compute units of the device (0: 256)
};

struct DecodeArgs {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* page_table;
    const int32_t* seq_lens;
    void* o;
    int B, Hq, Hkv, D, page_size;
    float scale;
    int window;     // 0: every cached token; W > 0: the W most recent
    int nsplit;     // context splits per (sequence, head group)
    float* ws;      // partial results, decode_workspace_floats() floats
    bool mfma;      // decode_on_mfma(): the MFMA kernel instead of the vector one
};

struct AppendArgs {
    const void* k_new;
    const void* v_new;
    void* k_pool;
    void* v_pool;
    const int32_t* page_table;
    const int32_t* seq_lens;
    int B, Hkv, D, page_size;
};

struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;   // [B, Hq, Sq] natural-log log-sum-exp from the forward pass
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv, Sq, Sk, D;
    float scale;
    int causal, window;
    void* ws;           // workspace of backward_workspace_bytes(..., kv_splits) bytes
    int num_cu = 0;     // compute units of the device (0: 256)
    int kv_splits = 1;  // backward_kv_splits(): runs per dK/dV key block
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

// Number of context splits for a decode call on a device with `num_cu`
// compute units, and the workspace (in floats) those splits need.
bool decode_on_mfma(int B, int Hq, int Hkv, int D, int num_cu);
int decode_nsplit(int B, int Hq, int Hkv, int num_cu, bool mfma);
size_t decode_workspace_floats(int B, int Hq, int D, int nsplit);
hipError_t launch_decode_paged(const DecodeArgs& a, hipStream_t stream);

// Allocation-free decode: a fixed 16 MiB device array per device holds the
// split partials. noalloc_scratch() returns its address on `device` (which
// must be current; looked up once per device) and the device's CU count.
constexpr size_t kNoallocScratchFloats = (size_t)4 << 20;
hipError_t noalloc_scratch(int device, float** ptr, int* num_cu);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
int backward_kv_splits(int B, int Hkv, int Sq, int Sk, int num_cu);
size_t backward_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv_splits);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);

}  // namespace attn
