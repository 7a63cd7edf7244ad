// Prefill attention forward in float32 throughout (accuracy path).
//
// Same operation as the bf16 kernel, O = softmax(mask(Q K^T * scale)) V with
// causal / sliding-window masks and GQA head sharing ("Attention 机制详解：
// 从 Self-Attention 到 Multi-Query Attention" §2.1–2.2 and §5.2), evaluated
// tile by tile with an online softmax (the pages' FlashAttention sections),
// but every operand and every product stays float32: no rounding of Q, K, P
// or V to a narrower type.
//
// Layout: a workgroup of 256 threads owns 64 query rows; four adjacent lanes
// share a row and split the head dimension d = part + 4x between them, so the
// four lanes read four consecutive floats of a staged K/V row (distinct LDS
// banks). 32-key tiles of K and V are staged through LDS; the partial dot
// products are summed across the four lanes with two lane exchanges.

#include "launch.h"

#include <cmath>

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;
constexpr int kBN = 32;

template <int D>
__global__ __launch_bounds__(kThreads)
void prefill_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                        const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                        int Hq, int Hkv, int Sq, int Sk, float c2, int causal, int window, int nqt) {
    constexpr int DP = D / 4;  // dims per lane
    __shared__ float ks[kBN][D];
    __shared__ float vs[kBN][D];

    const int item = blockIdx.x;
    const int qt = item % nqt;
    const int bh = item / nqt;
    const int h = bh % Hq;
    const int b = bh / Hq;
    const int g = h / (Hq / Hkv);

    const int tid = threadIdx.x;
    const int part = tid & 3;
    const int row = qt * kRows + (tid >> 2);
    const int off = Sk - Sq;
    const int pos = row + off;

    const size_t qo_base = ((size_t)b * Hq + h) * (size_t)Sq * D;
    const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)Sk * D;

    float q[DP], o[DP];
    const bool row_ok = row < Sq;
#pragma unroll
    for (int x = 0; x < DP; ++x) {
        q[x] = row_ok ? Q[qo_base + (size_t)row * D + part + 4 * x] : 0.f;
        o[x] = 0.f;
    }

    const int i0 = qt * kRows;
    const int row_end = min(i0 + kRows, Sq);
    const int hi = causal ? min(Sk, row_end - 1 + off + 1) : Sk;
    const int lo = (causal && window > 0) ? max(0, i0 + off - window + 1) : 0;

    float m_run = -INFINITY, l_run = 0.f;
    for (int j0 = (lo / kBN) * kBN; j0 < hi; j0 += kBN) {
        __syncthreads();
        for (int e = tid; e < kBN * D; e += kThreads) {
            const int jj = e / D, d = e % D;
            const int j = j0 + jj;
            ks[jj][d] = (j < Sk) ? K[kv_base + (size_t)j * D + d] : 0.f;
            vs[jj][d] = (j < Sk) ? V[kv_base + (size_t)j * D + d] : 0.f;
        }
        __syncthreads();

        float t[kBN];
        float mt = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kBN; ++jj) {
            float s = 0.f;
#pragma unroll
            for (int x = 0; x < DP; ++x) s = fmaf(q[x], ks[jj][part + 4 * x], s);
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            const int j = j0 + jj;
            bool ok = j < Sk;
            if (causal) ok = ok && j <= pos;
            if (window > 0) ok = ok && j > pos - window;
            t[jj] = ok ? s * c2 : -INFINITY;
            mt = fmaxf(mt, t[jj]);
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int x = 0; x < DP; ++x) o[x] *= alpha;
#pragma unroll
        for (int jj = 0; jj < kBN; ++jj) {
            const float p = exp2f(t[jj] - m_use);
            l_run += p;
#pragma unroll
            for (int x = 0; x < DP; ++x) o[x] = fmaf(p, vs[jj][part + 4 * x], o[x]);
        }
    }

    if (!row_ok) return;
    const float inv = 1.f / l_run;
    // log-sum-exp of the scaled logits, natural log (m_run in log2 units)
    if (LSE != nullptr && part == 0)
        LSE[((size_t)b * Hq + h) * Sq + row] = (m_run + log2f(l_run)) * 0.69314718055994531f;
#pragma unroll
    for (int x = 0; x < DP; ++x) O[qo_base + (size_t)row * D + part + 4 * x] = o[x] * inv;
}

template <int D>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
    const int nqt = (a.Sq + kRows - 1) / kRows;
    const long long grid = (long long)a.B * a.Hq * nqt;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const float c2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       a.Hq, a.Hkv, a.Sq, a.Sk, c2, a.causal, a.window, nqt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    return a.D == 128 ? launch_t<128>(a, stream) : launch_t<64>(a, stream);
}

}  // namespace attn
