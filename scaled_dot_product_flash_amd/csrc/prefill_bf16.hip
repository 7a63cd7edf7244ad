// Prefill attention forward, bfloat16 in/out, on gfx950 MFMA.
//
// What it computes: O = softmax(mask(Q K^T * scale)) V per (batch, query head),
// "Attention 机制详解：从 Self-Attention 到 Multi-Query Attention" §2.1–2.2,
// with GQA head sharing (§5.2: query head h reads K/V head h / (Hq/Hkv)),
// causal and sliding-window masks ("拆开 LLM（二）：手撕注意力", causal mask
// section; "LLM 核心技术：Attention 机制的实现与优化", SWA section).
//
// How: FlashAttention-style tiling with an online softmax (the pages'
// FlashAttention sections: blocks of Q, K, V are worked on on-chip, a running
// row maximum and row sum are kept, earlier partial output is rescaled when
// the maximum grows, and only O is written back).
//
// gfx950 mapping, per workgroup of 4 waves (256 threads):
//  * 128 query rows, 32 per wave. Each wave computes S^T = K_tile · Q^T with
//    v_mfma_f32_32x32x16_bf16, so a lane owns one query column and 16 key
//    rows of each 32-key block; the row maximum of a query is a reduction
//    over the lane's own values plus one exchange with lane ^ 32.
//  * Q lives in registers for the whole loop (it is the MFMA B operand).
//  * K tiles (key-major) and V tiles (stored transposed, d-major) are staged
//    through LDS, double buffered: the next tile's global loads are issued
//    before the current tile's MFMAs and written to the other buffer after.
//    16-byte chunks are XOR-swizzled by row so the MFMA operand reads
//    (32 rows at one column) hit distinct banks.
//  * O^T = V^T · P^T also runs on MFMA; P^T comes straight from the S^T
//    accumulators (converted to bf16 in registers) because the V^T tile is
//    stored with its keys permuted into the order the accumulator layout
//    hands them out (bits 2 and 3 of the key index swapped).
//  * Tiles wholly outside a wave's causal/window range are skipped; only
//    tiles that straddle a boundary or the key tail evaluate the mask.
//  * Work items are ordered (batch, kv head) major, then query tile from the
//    heaviest causal tile down, then the query heads of the group; each XCD
//    takes a contiguous run of items so the query heads sharing a K/V head
//    meet in the same L2.

#include "launch.h"

#include <cmath>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kXcds = 8;

template <int D> struct Tile { static constexpr int BN = (D == 128) ? 64 : 128; };

__device__ __forceinline__ uint4 ld_global16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// Position of key kappa (within a tile) in the transposed V tile: bits 2 and
// 3 swapped, so the 8 keys a lane contributes to one P^T·V MFMA k-step are
// adjacent and one 16-byte LDS read fetches them.
__device__ __forceinline__ int vt_pos(int kappa) {
    return (kappa & ~0xC) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}

template <int D, bool NEG>
__global__ __launch_bounds__(kThreads, 2)
void prefill_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                         const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                         int Hq, int Hkv, int Sq, int Sk, float c2, int causal, int window,
                         int nqt, int nitems, int per_xcd) {
    constexpr int BN = Tile<D>::BN;
    constexpr int KB = BN / 32;           // 32-key blocks per tile
    constexpr int KS = BN / 16;           // 16-key MFMA k-steps per tile (P·V)
    constexpr int DS = D / 16;            // 16-wide d steps (Q·K^T)
    constexpr int DB = D / 32;            // 32-row d blocks of O^T
    constexpr int CPR = D / 8;            // 16-byte chunks per K row
    constexpr int K_BYTES = BN * D * 2;
    constexpr int V_BYTES = D * BN * 2;
    constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    constexpr int KCH = BN * D / 8 / kThreads;  // K chunks per thread per tile
    static_assert(KCH * kThreads * 8 == BN * D, "K tile split");
    static_assert((BN / 4) * (D / 8) == kThreads, "V tile split");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF_BYTES];

    // ---- work item -------------------------------------------------------
    const int w = blockIdx.x;
    const int item = (w % kXcds) * per_xcd + w / kXcds;
    if (item >= nitems) return;
    const int G = Hq / Hkv;
    const int hg = item % G;
    const int r1 = item / G;
    const int qt = nqt - 1 - (r1 % nqt);
    const int bg = r1 / nqt;
    const int g = bg % Hkv;
    const int b = bg / Hkv;
    const int h = g * G + hg;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int ln = lane & 31;
    const int hh = lane >> 5;

    const int off = Sk - Sq;  // bottom-right causal alignment
    const int i0 = qt * kBM;
    const int row_end = min(i0 + kBM, Sq);

    const size_t qo_base = ((size_t)b * Hq + h) * (size_t)Sq * D;
    const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)Sk * D;
    const uint16_t* Kb = K + kv_base;
    const uint16_t* Vb = V + kv_base;

    // key range of the whole workgroup
    const int p_first = i0 + off;
    const int p_last = row_end - 1 + off;
    const int hi = causal ? min(Sk, p_last + 1) : Sk;
    const int lo = (causal && window > 0) ? max(0, p_first - window + 1) : 0;
    const int t_begin = lo / BN;
    const int t_end = (hi + BN - 1) / BN;

    // key range of this wave
    const int wr0 = i0 + 32 * wave;
    const int wr1 = min(wr0 + 32, Sq) - 1;
    const bool wave_rows = wr0 < Sq;
    const int wp0 = wr0 + off, wp1 = wr1 + off;
    const int w_hi = causal ? min(Sk - 1, wp1) : Sk - 1;           // largest visible key
    const int w_lo = (causal && window > 0) ? max(0, wp0 - window + 1) : 0;
    const int w_full_hi = causal ? min(Sk - 1, wp0) : Sk - 1;      // visible to every row
    const int w_full_lo = (causal && window > 0) ? max(0, wp1 - window + 1) : 0;

    // ---- Q in registers (MFMA B operand: column = query, 8 d per lane) ----
    const int qrow = wr0 + ln;
    const int qpos = qrow + off;
    bf16x8 qreg[DS];
    {
        const bool ok = qrow < Sq;
        const uint16_t* qp = Q + qo_base + (size_t)(ok ? qrow : 0) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            uint4 x = ok ? ld_global16(qp + 16 * s) : make_uint4(0, 0, 0, 0);
            qreg[s] = as_bf16x8(x);
        }
    }

    // ---- tile staging -----------------------------------------------------
    uint4 kreg[KCH];
    uint4 vreg[4];
    const int vm = tid % (BN / 4);   // V task: keys 4*vm .. 4*vm+3
    const int vc = tid / (BN / 4);   //         d   8*vc .. 8*vc+7

    auto load_tile = [&](int t) {
        const int j0 = t * BN;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int id = i * kThreads + tid;
            const int key = id / CPR, cc = id % CPR;
            const int j = j0 + key;
            kreg[i] = (j < Sk) ? ld_global16(Kb + (size_t)j * D + 8 * cc) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int j = j0 + 4 * vm + t4;
            vreg[t4] = (j < Sk) ? ld_global16(Vb + (size_t)j * D + 8 * vc) : make_uint4(0, 0, 0, 0);
        }
    };

    auto store_tile = [&](int buf) {
        unsigned char* kb = smem + buf * BUF_BYTES;
        unsigned char* vb = kb + K_BYTES;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int id = i * kThreads + tid;
            const int key = id / CPR, cc = id % CPR;
            *reinterpret_cast<uint4*>(kb + key * (D * 2) + ((cc ^ (key & 7)) << 4)) = kreg[i];
        }
        const int pos = vt_pos(4 * vm);
        const int chunk = pos >> 3;
        const int half8 = (pos & 7) * 2;  // 0 or 8 bytes into the chunk
        const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
        const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
        const uint32_t* x2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
        const uint32_t* x3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d0 = 8 * vc + 2 * e;
            const int d1 = d0 + 1;
            uint2 lo, hi2;
            lo.x = (x0[e] & 0xFFFFu) | (x1[e] << 16);
            lo.y = (x2[e] & 0xFFFFu) | (x3[e] << 16);
            hi2.x = (x0[e] >> 16) | (x1[e] & 0xFFFF0000u);
            hi2.y = (x2[e] >> 16) | (x3[e] & 0xFFFF0000u);
            *reinterpret_cast<uint2*>(vb + d0 * (BN * 2) + ((chunk ^ (d0 & 7)) << 4) + half8) = lo;
            *reinterpret_cast<uint2*>(vb + d1 * (BN * 2) + ((chunk ^ (d1 & 7)) << 4) + half8) = hi2;
        }
    };

    // ---- running state ------------------------------------------------------
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m_run = -INFINITY;  // running max of scaled logits, log2 units
    float l_run = 0.f;        // this lane's share of the running row sum

    load_tile(t_begin);
    store_tile(0);
    __syncthreads();

    for (int t = t_begin; t < t_end; ++t) {
        const int cur = (t - t_begin) & 1;
        const bool has_next = t + 1 < t_end;
        if (has_next) load_tile(t + 1);
        const int j0 = t * BN;
        const bool active = wave_rows && j0 <= w_hi && j0 + BN - 1 >= w_lo;
        if (active) {
            const unsigned char* kb = smem + cur * BUF_BYTES;
            const unsigned char* vb = kb + K_BYTES;

            // S^T = K_tile · Q^T, 32 keys x 32 queries per accumulator
            f32x16 sacc[KB];
#pragma unroll
            for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[kbk][v] = 0.f;
#pragma unroll
            for (int s = 0; s < DS; ++s) {
#pragma unroll
                for (int kbk = 0; kbk < KB; ++kbk) {
                    const int key = 32 * kbk + ln;
                    const int cc = 2 * s + hh;
                    const uint4 a = *reinterpret_cast<const uint4*>(kb + key * (D * 2) + ((cc ^ (key & 7)) << 4));
                    sacc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qreg[s], sacc[kbk], 0, 0, 0);
                }
            }

            // mask (boundary tiles only) and the tile's extreme raw logit
            const bool edge = (j0 + BN - 1 > w_full_hi) || (j0 < w_full_lo);
            const float masked = NEG ? INFINITY : -INFINITY;
            uint64_t vis = ~0ull;
            float mx = masked;
            if (edge) {
                vis = 0;
#pragma unroll
                for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int j = j0 + 32 * kbk + 8 * (v >> 2) + 4 * hh + (v & 3);
                        bool ok = j < Sk;
                        if (causal) ok = ok && j <= qpos;
                        if (window > 0) ok = ok && j > qpos - window;
                        vis |= (uint64_t)ok << (16 * kbk + v);
                        const float x = ok ? sacc[kbk][v] : masked;
                        mx = NEG ? fminf(mx, x) : fmaxf(mx, x);
                    }
            } else {
#pragma unroll
                for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        mx = NEG ? fminf(mx, sacc[kbk][v]) : fmaxf(mx, sacc[kbk][v]);
            }
            const float other = xor32(mx);
            mx = NEG ? fminf(mx, other) : fmaxf(mx, other);

            // online softmax update (log2 domain: exp(x) = exp2(x * log2 e))
            const float mt = (mx == masked) ? -INFINITY : mx * c2;
            const float m_new = fmaxf(m_run, mt);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run - m_use);
            m_run = m_new;

            float lsum = 0.f;
#pragma unroll
            for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    float p = __builtin_amdgcn_exp2f(fmaf(sacc[kbk][v], c2, -m_use));
                    if (edge) p = ((vis >> (16 * kbk + v)) & 1) ? p : 0.f;
                    sacc[kbk][v] = p;
                    lsum += p;
                }
            l_run = l_run * alpha + lsum;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;

            // P^T as bf16 B operands, straight from the accumulators
            bf16x8 pb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    f32x2 pr = {sacc[ks >> 1][8 * (ks & 1) + j], sacc[ks >> 1][8 * (ks & 1) + j + 1]};
                    bf16x2 pbf = __builtin_convertvector(pr, bf16x2);
                    pb[ks][j] = pbf[0];
                    pb[ks][j + 1] = pbf[1];
                }
            }

            // O^T += V^T · P^T
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int d = 32 * db + ln;
                    const int q8 = 2 * ks + hh;
                    const uint4 a = *reinterpret_cast<const uint4*>(vb + d * (BN * 2) + ((q8 ^ (d & 7)) << 4));
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb[ks], oacc[db], 0, 0, 0);
                }
            }
        }
        if (has_next) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, bf16, 4 consecutive d per 8-byte store -----
    if (!wave_rows || qrow >= Sq) return;
    const float l_tot = l_run + xor32(l_run);
    const float inv = 1.f / l_tot;
    uint16_t* op = O + qo_base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x2 a = {oacc[db][4 * r + 0] * inv, oacc[db][4 * r + 1] * inv};
            f32x2 c = {oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv};
            bf16x2 x = __builtin_convertvector(a, bf16x2);
            bf16x2 y = __builtin_convertvector(c, bf16x2);
            uint2 st;
            st.x = __builtin_bit_cast(uint32_t, x);
            st.y = __builtin_bit_cast(uint32_t, y);
            *reinterpret_cast<uint2*>(op + 32 * db + 8 * r + 4 * hh) = st;
        }
}

template <int D, bool NEG>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
    const int nqt = (a.Sq + kBM - 1) / kBM;
    const long long nitems = (long long)a.B * a.Hq * nqt;
    const long long per_xcd = (nitems + kXcds - 1) / kXcds;
    const long long grid = per_xcd * kXcds;
    if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const float c2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, NEG>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                       a.Hq, a.Hkv, a.Sq, a.Sk, c2, a.causal, a.window, nqt, (int)nitems, (int)per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const bool neg = a.scale < 0.f;
    if (a.D == 128) return neg ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return neg ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace attn
