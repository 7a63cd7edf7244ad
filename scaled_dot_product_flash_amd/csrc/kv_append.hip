// Append the new token's k and v to a paged KV cache, bfloat16, gfx950.
//
// The decode step of "拆开 LLM（二）：手撕注意力" (KV-cache section) first
// appends the new token's key and value to the cache and then lets the token
// attend to every cached position; with the paged layout of "LLM 核心技术：
// Attention 机制的实现与优化" (PagedAttention section) the append is a write
// into the slot of the sequence's last logical page. seq_lens[b] already
// counts the new token, so it lands at position t = seq_lens[b] - 1: slot
// t % page_size of physical page page_table[off_b + t / page_size], with
// off_b the same prefix sum over ceil(seq_lens[j] / page_size) that the decode
// kernel uses.
//
// One workgroup per sequence. The prefix sum is a strided partial sum plus a
// wave reduction; then each lane copies 16-byte chunks of k and v. The work is
// a few KiB per sequence, so the kernel is bound by launch latency, not HBM.

#include "launch.h"
#include "paging.h"

namespace attn {
namespace {

constexpr int kThreads = 128;

__global__ __launch_bounds__(kThreads)
void kv_append_kernel(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                      uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                      const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
                      int Hkv, int D, int ps_log2) {
    __shared__ int sh_part[kThreads / 64];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int ps = 1 << ps_log2;

    int part = 0;
    for (int j = tid; j < b; j += kThreads) part += seq_pages(lens[j], ps_log2);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if ((tid & 63) == 0) sh_part[tid >> 6] = part;
    __syncthreads();
    int off_b = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) off_b += sh_part[w];

    const int t = lens[b] - 1;
    // outside the precondition seq_lens[b] >= 1: there is no position to
    // write, and t = -1 would address the table entry before the sequence's
    // own (another sequence's last page)
    if (t < 0) return;
    const int page = table[off_b + (t >> ps_log2)];
    const size_t dst = pool_tile(page, 0, Hkv, ps_log2, D) + (size_t)(t & (ps - 1)) * D;  // head 0 of the slot
    const size_t head_stride = (size_t)ps * D;
    const int chunks = D / 8;                      // 16-byte chunks per head row
    for (int i = tid; i < Hkv * chunks; i += kThreads) {
        const int g = i / chunks, c = i % chunks;
        const size_t src = ((size_t)b * Hkv + g) * D + 8 * c;
        const size_t d = dst + g * head_stride + 8 * c;
        *reinterpret_cast<uint4*>(k_pool + d) = *reinterpret_cast<const uint4*>(k_new + src);
        *reinterpret_cast<uint4*>(v_pool + d) = *reinterpret_cast<const uint4*>(v_new + src);
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    int ps_log2 = 0;
    while ((1 << ps_log2) < a.page_size) ++ps_log2;
    if (log_enabled())
        log_dispatch("kv_append_kernel B=%d Hkv=%d D=%d page_size=%d: grid %d x %d threads", a.B, a.Hkv, a.D,
                     a.page_size, a.B, kThreads);
    hipLaunchKernelGGL(kv_append_kernel, dim3(a.B), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.k_new, (const uint16_t*)a.v_new, (uint16_t*)a.k_pool,
                       (uint16_t*)a.v_pool, a.page_table, a.seq_lens, a.Hkv, a.D, ps_log2);
    return hipGetLastError();
}

}  // namespace attn
