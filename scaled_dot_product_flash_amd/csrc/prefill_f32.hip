// Prefill attention forward in float32 throughout (accuracy path).
//
// Same operation as the bf16 kernel, O = softmax(mask(Q K^T * scale)) V with
// causal / sliding-window masks and GQA head sharing ("Attention 机制详解：
// 从 Self-Attention 到 Multi-Query Attention" §2.1–2.2 and §5.2), evaluated
// tile by tile with an online softmax (the pages' FlashAttention sections),
// but every operand and every product stays float32: no rounding of Q, K, P
// or V to a narrower type.
//
// Layout: a workgroup of four waves owns 16 query rows; in every wave four
// adjacent lanes share a row and split the head dimension into four
// contiguous quarters (d = part * D/4 + x), so a lane reads its quarter of a
// staged K/V row with 16-byte LDS reads (the rows of a wave read the same key:
// broadcast). The four waves take every fourth 16-key tile of the row block's
// key range, each with its own online softmax over its tiles and its own LDS
// tiles, and their (max, sum, output) partials are merged at the end with the
// same rescale rule; this cuts the serial chain of a row by four for short
// sequences. The partial dot products are summed across the four lanes of a
// row with two DPP lane exchanges.

#include "launch.h"

#include <cmath>

namespace attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;   // query rows per workgroup: four lanes per row in each wave
constexpr int kBN = 16;     // keys per staged tile of one wave

// Sums over the four lanes of a row through DPP quad permutations (lane ^ 1,
// lane ^ 2) instead of LDS-routed shuffles: a VALU operand modifier, no LDS
// round trip per key.
__device__ __forceinline__ float quad_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

template <int D>
__global__ __launch_bounds__(kThreads)
void prefill_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                        const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                        int Hq, int Hkv, int Sq, int Sk, float c2, int causal, int window, int nqt) {
    constexpr int DP = D / 4;  // dims per lane: part * DP .. part * DP + DP - 1 (16-byte LDS reads)
    // per wave: its K and V tiles; after the key loop, its (m, l, o) partials
    __shared__ __attribute__((aligned(16))) float ks[kWaves][kBN][D];
    __shared__ __attribute__((aligned(16))) float vs[kWaves][kBN][D];

    const int item = blockIdx.x;
    const int qt = item % nqt;
    const int bh = item / nqt;
    const int h = bh % Hq;
    const int b = bh / Hq;
    const int g = h / (Hq / Hkv);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int part = lane & 3;
    const int row = qt * kRows + (lane >> 2);
    const int off = Sk - Sq;
    const int pos = row + off;

    const size_t qo_base = ((size_t)b * Hq + h) * (size_t)Sq * D;
    const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)Sk * D;

    float q[DP], o[DP];
    const bool row_ok = row < Sq;
#pragma unroll
    for (int x = 0; x < DP; ++x) {
        q[x] = row_ok ? Q[qo_base + (size_t)row * D + part * DP + x] : 0.f;
        o[x] = 0.f;
    }

    const int i0 = qt * kRows;
    const int row_end = min(i0 + kRows, Sq);
    const int hi = causal ? min(Sk, row_end - 1 + off + 1) : Sk;
    const int lo = (causal && window > 0) ? max(0, i0 + off - window + 1) : 0;

    // the four waves take every fourth key tile of the workgroup's range and
    // keep their own online softmax; the partials are merged at the end
    float m_run = -INFINITY, l_run = 0.f;
    float (*kw)[D] = ks[wave];
    float (*vw)[D] = vs[wave];
    for (int j0 = (lo / kBN + wave) * kBN; j0 < hi; j0 += kWaves * kBN) {
        // this wave's tile: 64 lanes stage kBN x D floats of K and V
        for (int e = lane * 4; e < kBN * D; e += 64 * 4) {
            const int jj = e / D, d = e % D;
            const int j = j0 + jj;
            const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4*>(&kw[jj][d]) =
                (j < Sk) ? *reinterpret_cast<const float4*>(K + kv_base + (size_t)j * D + d) : zero;
            *reinterpret_cast<float4*>(&vw[jj][d]) =
                (j < Sk) ? *reinterpret_cast<const float4*>(V + kv_base + (size_t)j * D + d) : zero;
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

        float t[kBN];
        float mt = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kBN; ++jj) {
            float s = 0.f;
#pragma unroll
            for (int x = 0; x < DP; ++x) s = fmaf(q[x], kw[jj][part * DP + x], s);
            s += quad_xor1(s);
            s += quad_xor2(s);
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
            for (int x = 0; x < DP; ++x) o[x] = fmaf(p, vw[jj][part * DP + x], o[x]);
        }
        // the next tile overwrites this one: finish reading it first
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
    }

    // merge the four waves' partials (m, l, o) with the online-softmax rule:
    // m = max m_w, l = sum 2^(m_w - m) l_w, o = sum 2^(m_w - m) o_w
    __syncthreads();
    float* part_o = &ks[wave][0][0];             // 16 rows x 4 lanes x DP floats
    float* part_ml = &vs[wave][0][0];            // 16 rows x 4 lanes x 2 floats
#pragma unroll
    for (int x = 0; x < DP; ++x) part_o[lane * DP + x] = o[x];
    part_ml[lane * 2] = m_run;
    part_ml[lane * 2 + 1] = l_run;
    __syncthreads();
    if (wave != 0 || !row_ok) return;
    float mw[kWaves], m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        mw[w] = (&vs[w][0][0])[lane * 2];
        m = fmaxf(m, mw[w]);
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int x = 0; x < DP; ++x) o[x] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float a = exp2f(mw[w] - m_use);   // 0 for a wave that saw no visible key
        l += a * (&vs[w][0][0])[lane * 2 + 1];
#pragma unroll
        for (int x = 0; x < DP; ++x) o[x] = fmaf(a, (&ks[w][0][0])[lane * DP + x], o[x]);
    }
    const float inv = 1.f / l;
    // log-sum-exp of the scaled logits, natural log (m in log2 units)
    if (LSE != nullptr && part == 0)
        LSE[((size_t)b * Hq + h) * Sq + row] = (m + log2f(l)) * 0.69314718055994531f;
#pragma unroll
    for (int x = 0; x < DP; ++x) O[qo_base + (size_t)row * D + part * DP + x] = o[x] * inv;
}

template <int D>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
    const int nqt = (a.Sq + kRows - 1) / kRows;
    const long long grid = (long long)a.B * a.Hq * nqt;
    if (!grid_fits(grid, kThreads)) return hipErrorInvalidValue;
    const float c2 = a.scale * 1.4426950408889634f;
    if (log_enabled())
        log_dispatch("prefill_f32_kernel<%d> B=%d Hq=%d Hkv=%d Sq=%d Sk=%d causal=%d window=%d%s: grid %lld x %d "
                     "threads, %d rows per workgroup", D, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.causal, a.window,
                     a.lse ? " +lse" : "", grid, kThreads, kRows);
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
