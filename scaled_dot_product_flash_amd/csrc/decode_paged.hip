// Single-token decode over a paged KV cache, bfloat16, gfx950.
//
// What it computes: for each sequence b and query head h,
//   o[b,h] = softmax(q[b,h] · K_b^T * scale) V_b
// over every cached token 0 .. seq_lens[b]-1, with no mask ("拆开 LLM（二）：
// 手撕注意力", KV-cache section: the new token attends to all cached
// positions). K_b / V_b are not contiguous: token t of sequence b is slot
// t % page_size of physical page page_table[off_b + t / page_size] of a
// global pool ("LLM 核心技术：Attention 机制的实现与优化", PagedAttention
// section; "Attention From Scratch", paged-KV-cache part: fixed-size pages, a
// per-sequence page table and a global page pool).
//
// The step is bound by HBM bandwidth (every cached K/V byte is read once), so
// the design is about bytes in flight and cheap per-byte VALU work. Fewer than 8
// query heads per K/V head take the vector kernel below; 8 and more, whose
// per-byte dot products would bound the vector kernel, take the MFMA kernel
// further down (described there). Both write the same split partials.
// The vector kernel:
//  * Split kernel, grid (split, kv-head group, sequence). The query heads that
//    share a K/V head (up to 8) are packed into one workgroup so each page is
//    read once for all of them. The sequence's context is cut into `nsplit`
//    contiguous runs of 16-token (D=128) or 32-token (D=64) blocks; the four
//    waves of a workgroup take the run's blocks round-robin. Grid slot z takes
//    the sequence of z-th largest length (up to 256 sequences), so the
//    longest work is dispatched first and the tail of the grid is short.
//  * A block is read with four 16-byte loads per lane per tensor; lane l holds
//    d-chunk l % (D/8) of token l / (D/8) (+ 4 or 8 per load), so every load
//    instruction reads 1 KiB of one page contiguously. The next block's loads
//    are issued before the current block is consumed.
//  * q·k: bf16 pair dot products (v_dot2_f32_bf16) over the lane's 8 dims,
//    then a DPP all-reduce over the lanes of the token.
//  * Online softmax per lane row (the lanes that hold the same tokens): the
//    running max / sum / output of a row only ever see that row's tokens, so
//    the loop needs no cross-row traffic; rows, then waves, then splits are
//    merged at the end with the same rescale rule the online softmax uses.
//  * p·v: P is rounded to bf16 and paired over two tokens, V is re-paired over
//    the same two tokens, and v_dot2_f32_bf16 accumulates both at once.
//  * Tokens at or past seq_lens[b] are excluded by selection (logit -inf, V
//    zeroed), never by multiplying with 0, so NaN padding cannot leak.
//  * Sliding window (window W > 0): only the W most recent tokens, positions
//    len-W .. len-1, are visible ("拆开 LLM（二）：手撕注意力", exercise that keeps
//    the last 256 cache entries; "LLM 核心技术：Attention 机制的实现与优化",
//    sliding-window section); the splits cover just those blocks and tokens
//    before len-W in the first block are excluded the same way.
//  * Merge kernel: per (sequence, query head) combines the split partials
//    (m, l, o) into the bf16 output.

#include "launch.h"
#include "paging.h"

#include <cmath>

namespace attn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the lanes that hold one token, for N independent values at once:
// 16 lanes (a DPP row) for D = 128, 8 lanes (half a row) for D = 64. Every
// lane of the group ends with the sums. Each step is applied to all N values
// before the next, so no value waits on its own previous DPP result.
template <int CPT, int N>
__device__ __forceinline__ void token_sum_all(float* x) {
    if constexpr (CPT == 16) {
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] += dpp<0x128>(x[n]);  // row_ror:8
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] += dpp<0x124>(x[n]);  // row_ror:4
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] += dpp<0x122>(x[n]);  // row_ror:2
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] += dpp<0x121>(x[n]);  // row_ror:1
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] += dpp<0x141>(x[n]);  // row_half_mirror: lane i + lane 7-i
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] += dpp<0xB1>(x[n]);   // quad_perm [1,0,3,2]
#pragma unroll
        for (int n = 0; n < N; ++n) x[n] += dpp<0x4E>(x[n]);   // quad_perm [2,3,0,1]
    }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint4 ld16_nt(const uint16_t* p) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

// Lazy-rescale threshold for the reference maximum, log2 units.
constexpr float kLazy = 8.0f;
constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)

template <int D, int GH, bool NEG>
__global__ __launch_bounds__(kThreads)
void decode_split_kernel(const uint16_t* __restrict__ Qp, const uint16_t* __restrict__ Kp,
                         const uint16_t* __restrict__ Vp, const int32_t* __restrict__ table,
                         const int32_t* __restrict__ lens, float* __restrict__ ws,
                         int Hq, int Hkv, int ps_log2, int nsplit, float c2, int window) {
    constexpr int CPT = D / 8;        // lanes per token (16-byte chunks per row)
    constexpr int TPI = 64 / CPT;     // tokens per load instruction
    constexpr int TB = 4 * TPI;       // tokens per block

    __shared__ float sh_m[kWaves][GH];
    __shared__ float sh_l[kWaves][GH];
    __shared__ __attribute__((aligned(16))) float sh_o[kWaves][GH][D];
    __shared__ int sh_red[kWaves];

    const int split = blockIdx.x;
    const int hgrp = blockIdx.y;        // (kv head, head group)
    __shared__ int sh_len[kThreads];
    __shared__ int sh_b;
    int b = blockIdx.z;
    {
        // longest sequences first: slot z of the grid takes the sequence of
        // length rank z (ties by index), so the long work items start early
        const int B = gridDim.z;
        if (B <= kThreads) {
            if ((int)threadIdx.x < B) sh_len[threadIdx.x] = lens[threadIdx.x];
            __syncthreads();
            if ((int)threadIdx.x < B) {
                const int my = sh_len[threadIdx.x];
                int rank = 0;
                for (int j = 0; j < B; ++j) {
                    const int lj = sh_len[j];
                    rank += (lj > my) || (lj == my && j < (int)threadIdx.x);
                }
                if (rank == (int)blockIdx.z) sh_b = threadIdx.x;
            }
            __syncthreads();
            b = sh_b;
        }
    }
    const int G = Hq / Hkv;
    const int groups_per_kv = G / GH;
    const int g = hgrp / groups_per_kv;
    const int h0 = g * G + (hgrp % groups_per_kv) * GH;
    const int ps = 1 << ps_log2;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane % CPT;
    const int r = lane / CPT;

    // off_b = sum_{j<b} ceil(len_j / ps), the sequence's first page-table entry
    int part = 0;
    for (int j = tid; j < b; j += kThreads) part += seq_pages(lens[j], ps_log2);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (lane == 0) sh_red[wave] = part;
    __syncthreads();
    const int off_b = sh_red[0] + sh_red[1] + sh_red[2] + sh_red[3];
    const int len = lens[b];
    const int32_t* tab = table + off_b;

    // visible tokens first .. len-1; this split's blocks [blk_begin, blk_end)
    const int first = window_first(len, window);
    const UnitRun run = split_units(first, len, TB, split, nsplit);
    const int blk_begin = run.begin, blk_end = run.end;

    // q of the packed heads: 8 dims (4 bf16 pairs) per lane and head
    uint32_t qv[GH][4];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        const uint4 x = ld16(Qp + ((size_t)b * Hq + h0 + j) * D + 8 * c);
        qv[j][0] = x.x; qv[j][1] = x.y; qv[j][2] = x.z; qv[j][3] = x.w;
    }

    float m_run[GH], l_run[GH], o[GH][8];
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
    }

    // K/V pages are streamed once per decode step: nontemporal loads keep them
    // from displacing other data in the caches. The page base is wave-uniform
    // (scalar), the lane's offset inside the (page, head) tile is 32-bit.
    const int lane_off = r * D + 8 * c;
    auto load_block = [&](int blk, uint4 (&kx)[4], uint4 (&vx)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t0 = blk * TB + i * TPI;           // first token of this load
            if (t0 < len) {
                const int page = __builtin_amdgcn_readfirstlane(tab[t0 >> ps_log2]);
                const size_t tile = pool_tile(page, g, Hkv, ps_log2, D) + (size_t)(t0 & (ps - 1)) * D;
                kx[i] = ld16_nt(Kp + tile + lane_off);
                vx[i] = ld16_nt(Vp + tile + lane_off);
            } else {
                kx[i] = make_uint4(0, 0, 0, 0);
                vx[i] = make_uint4(0, 0, 0, 0);
            }
        }
    };

    // one 16/32-token block already in registers: logits, online softmax, P·V
    auto process = [&](int blk, const uint4 (&kc)[4], uint4 (&vc)[4]) {
        // raw logits q.k of the lane's 4 tokens for every packed head; the
        // 4*GH dot products and their lane sums advance in lock-step so that
        // independent instructions sit between the dependent DPP steps
        float s[4][GH];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < GH; ++j) s[i][j] = dot2(qv[j][0], kc[i].x, 0.f);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < GH; ++j) s[i][j] = dot2(qv[j][1], kc[i].y, s[i][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < GH; ++j) s[i][j] = dot2(qv[j][2], kc[i].z, s[i][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < GH; ++j) s[i][j] = dot2(qv[j][3], kc[i].w, s[i][j]);
        token_sum_all<CPT, 4 * GH>(&s[0][0]);

        // blocks at either end of the visible range: tokens at or past len, or
        // before the window, get an extreme logit that never wins the max, and
        // their V rows become zeros
        const bool partial = (blk + 1) * TB > len || blk * TB < first;
        bool ok[4] = {true, true, true, true};
        if (partial) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = blk * TB + i * TPI + r;
                ok[i] = tok < len && tok >= first;
                if (!ok[i]) {
#pragma unroll
                    for (int j = 0; j < GH; ++j) s[i][j] = NEG ? INFINITY : -INFINITY;
                    vc[i] = make_uint4(0, 0, 0, 0);
                }
            }
        }

        // V re-paired over tokens (0,1) and (2,3) for the bf16 pair products
        uint32_t vlo01[4], vhi01[4], vlo23[4], vhi23[4];
        const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vc[0]);
        const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vc[1]);
        const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&vc[2]);
        const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&vc[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vlo01[e] = (v0[e] & 0xFFFFu) | (v1[e] << 16);
            vhi01[e] = (v0[e] >> 16) | (v1[e] & 0xFFFF0000u);
            vlo23[e] = (v2[e] & 0xFFFFu) | (v3[e] << 16);
            vhi23[e] = (v2[e] >> 16) | (v3[e] & 0xFFFF0000u);
        }

#pragma unroll
        for (int j = 0; j < GH; ++j) {
            // this lane row's extreme raw logit -> scaled maximum (log2 units)
            const float mx = NEG ? fminf(fminf(s[0][j], s[1][j]), fminf(s[2][j], s[3][j]))
                                 : fmaxf(fmaxf(s[0][j], s[1][j]), fmaxf(s[2][j], s[3][j]));
            const float mt = (mx == (NEG ? INFINITY : -INFINITY)) ? -INFINITY : mx * c2;
            // lazy reference maximum: move it only when exceeded by kLazy, so
            // p <= 2^kLazy and o is rescaled rarely (same reference in o and l)
            const bool need = mt > m_run[j] + kLazy;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float alpha = need ? __builtin_amdgcn_exp2f(m_run[j] - mt) : 1.f;
                m_run[j] = need ? mt : m_run[j];
                l_run[j] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
            }
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(s[i][j], c2, -m_run[j]));
            if (partial) {
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = ok[i] ? p[i] : 0.f;
            }
            const uint32_t p01 = pack_bf16(p[0], p[1]);
            const uint32_t p23 = pack_bf16(p[2], p[3]);
            // l sums the same bf16-rounded probabilities that weight V
            l_run[j] = dot2(p23, kOnes, dot2(p01, kOnes, l_run[j]));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[j][2 * e] = dot2(p23, vlo23[e], dot2(p01, vlo01[e], o[j][2 * e]));
                o[j][2 * e + 1] = dot2(p23, vhi23[e], dot2(p01, vhi01[e], o[j][2 * e + 1]));
            }
        }
    };

    // software pipeline over this wave's blocks (blk_begin + wave, + 4, ...):
    // the next block's loads are in flight while the current one is consumed;
    // two register sets alternate so no copies are needed
    uint4 kA[4], vA[4], kB[4], vB[4];
    int blk = blk_begin + wave;
    if (blk < blk_end) load_block(blk, kA, vA);
    while (blk < blk_end) {
        int next = blk + kWaves;
        if (next < blk_end) load_block(next, kB, vB);
        process(blk, kA, vA);
        blk = next;
        if (blk >= blk_end) break;
        next = blk + kWaves;
        if (next < blk_end) load_block(next, kA, vA);
        process(blk, kB, vB);
        blk = next;
    }

    // merge the lane rows of the wave (rows differ in lane bits >= log2(CPT))
#pragma unroll
    for (int j = 0; j < GH; ++j) {
        float M = m_run[j];
#pragma unroll
        for (int x = CPT; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
        const float M_use = (M == -INFINITY) ? 0.f : M;
        const float sc = exp2f(m_run[j] - M_use);
        float L = l_run[j] * sc;
#pragma unroll
        for (int x = CPT; x < 64; x <<= 1) L += __shfl_xor(L, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = o[j][e] * sc;
#pragma unroll
            for (int x = CPT; x < 64; x <<= 1) v += __shfl_xor(v, x);
            o[j][e] = v;
        }
        if (r == 0) {
            *reinterpret_cast<float4*>(&sh_o[wave][j][8 * c]) = make_float4(o[j][0], o[j][1], o[j][2], o[j][3]);
            *reinterpret_cast<float4*>(&sh_o[wave][j][8 * c + 4]) = make_float4(o[j][4], o[j][5], o[j][6], o[j][7]);
        }
        if (lane == 0) {
            sh_m[wave][j] = M;
            sh_l[wave][j] = L;
        }
    }
    __syncthreads();

    // merge the waves and write this split's partial (m, l, o) per head
    for (int idx = tid; idx < GH * D; idx += kThreads) {
        const int j = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh_m[w][j]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = exp2f(sh_m[w][j] - M_use);
            L += sh_l[w][j] * sc;
            acc += sh_o[w][j][d] * sc;
        }
        const size_t unit = ((size_t)b * Hq + h0 + j) * nsplit + split;
        ws[unit * D + d] = acc;
        if (d == 0) {
            float* ml = ws + (size_t)gridDim.z * Hq * nsplit * D;
            ml[2 * unit] = M;
            ml[2 * unit + 1] = L;
        }
    }
}

template <int D>
__global__ __launch_bounds__(D)
void decode_merge_kernel(const float* __restrict__ ws, uint16_t* __restrict__ Op, int B, int Hq, int nsplit) {
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ml = ws + (size_t)B * Hq * nsplit * D;
    const size_t u0 = (size_t)bh * nsplit;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * (u0 + s)]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float sc = exp2f(ml[2 * (u0 + s)] - M_use);
        L += ml[2 * (u0 + s) + 1] * sc;
        acc += ws[(u0 + s) * D + d] * sc;
    }
    const float out = acc / L;
    const __bf16 ob = (__bf16)out;
    Op[(size_t)bh * D + d] = __builtin_bit_cast(uint16_t, ob);
}

// ---- decode on the matrix cores ---------------------------------------------
//
// The query heads that share a K/V head form a small dense contraction with
// the cached tokens: S^T (tokens x heads) = K Q^T and O^T (dims x heads) +=
// V^T P^T. With up to 32 heads as the 32 columns of v_mfma_f32_32x32x16_bf16
// the vector ALU is left with the softmax only. The launcher takes this kernel
// for 8 and more heads per K/V head, where the vector kernel above is bound by
// its dot products and lane sums.
//  * Grid (split, kv head x head group of <= 32, sequence by length rank);
//    a split's 32-token tiles are dealt round-robin to the four waves, each
//    with its own online softmax; the waves merge at the end and the split's
//    partial (m, l, o) goes to the same workspace as the vector kernel's.
//  * K tiles go from HBM straight into registers in the MFMA operand layout
//    (lane%32 = token, 8-dim chunks), one tile ahead of use; V tiles go by
//    buffer->LDS DMA into two LDS stages per wave and are read back with the
//    transposing LDS read as the V^T operand. Page ids are scalar loads, so
//    waiting for them never waits for the K/V loads in flight. With two
//    stages the kernel fits two workgroups per CU at D = 128 (207 VGPRs,
//    66 KB of LDS) and four at D = 64: more independent waves hide the load
//    latency better than deeper stages in one workgroup per CU did.
//  * Every step issues the same instructions: tokens past the length are
//    clamped to the last token for the K loads (valid memory, masked logits)
//    and read as zeros for V (range check), and past a wave's last tile the
//    issue is a dummy (K from the last token, which the cache holds; V from a
//    zero-size range, no memory traffic). The compiler then counts the loads
//    between a tile's issue and its use exactly and waits for that tile only.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource word 3, gfx9 family
constexpr int kTT = 32;                  // tokens per tile

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

template <int D, bool NEG>
__global__ __launch_bounds__(kThreads, 2)
void decode_mfma_kernel(const uint16_t* __restrict__ Qp, const uint16_t* __restrict__ Kp,
                        const uint16_t* __restrict__ Vp, const int32_t* __restrict__ table,
                        const int32_t* __restrict__ lens, float* __restrict__ ws,
                        int Hq, int Hkv, int ps_log2, int nsplit, float c2, int window) {
    constexpr int DS = D / 16;          // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;          // 32-dim blocks of O^T
    constexpr int KS = kTT / 16;        // k-steps of O^T += V^T P^T
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int RPS = 64 / CPR;       // rows per 1 KiB DMA slot
    constexpr int VT = kTT * D * 2;     // bytes of a V tile
    constexpr int VSLOTS = VT / 1024;
    // one LDS object per stage (four waves' tiles each), so that the
    // compiler's wait for DMA into LDS can tell the stages apart
    __shared__ __attribute__((aligned(16))) unsigned char vl0[kWaves * VT];
    __shared__ __attribute__((aligned(16))) unsigned char vl1[kWaves * VT];
    __shared__ float sh_m[kWaves * 32];
    __shared__ float sh_l[kWaves * 32];
    __shared__ int sh_len[kThreads];
    __shared__ int sh_b;
    __shared__ int sh_red[kWaves];

    const int split = blockIdx.x;
    const int tid = threadIdx.x;
    int b = blockIdx.z;
    {
        // longest sequences first: slot z of the grid takes the sequence of
        // length rank z (ties by index)
        const int B = gridDim.z;
        if (B <= kThreads) {
            if (tid < B) sh_len[tid] = lens[tid];
            __syncthreads();
            if (tid < B) {
                const int my = sh_len[tid];
                int rank = 0;
                for (int j = 0; j < B; ++j) {
                    const int lj = sh_len[j];
                    rank += (lj > my) || (lj == my && j < tid);
                }
                if (rank == (int)blockIdx.z) sh_b = tid;
            }
            __syncthreads();
            b = __builtin_amdgcn_readfirstlane(sh_b);
        }
    }
    const int G = Hq / Hkv;
    const int ngrp = (G + 31) >> 5;
    const int g = blockIdx.y / ngrp;
    const int hg0 = (blockIdx.y % ngrp) * 32;
    const int GC = min(32, G - hg0);            // heads of this group
    const int h0 = g * G + hg0;
    const int ps = 1 << ps_log2;

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int ln = lane & 31;
    const int hh = lane >> 5;

    // off_b = sum_{j<b} ceil(len_j / ps), the sequence's first page-table entry
    int part = 0;
    for (int j = tid; j < b; j += kThreads) part += seq_pages(lens[j], ps_log2);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (lane == 0) sh_red[wave] = part;
    __syncthreads();
    const int off_b = __builtin_amdgcn_readfirstlane(sh_red[0] + sh_red[1] + sh_red[2] + sh_red[3]);
    const int len = __builtin_amdgcn_readfirstlane(lens[b]);
    const int32_t* tab = table + off_b;
    const int last_page = (len - 1) >> ps_log2;

    if (len < 1) {
        // outside the precondition (a sequence owns no page): an empty partial,
        // as the vector kernel leaves; no load is issued
        for (int idx = tid; idx < GC * D; idx += kThreads) {
            const int j = idx / D, d = idx % D;
            const size_t unit = ((size_t)b * Hq + h0 + j) * nsplit + split;
            ws[unit * D + d] = 0.f;
            if (d == 0) {
                float* ml = ws + (size_t)gridDim.z * Hq * nsplit * D;
                ml[2 * unit] = -INFINITY;
                ml[2 * unit + 1] = 0.f;
            }
        }
        return;
    }

    // this split's tiles of the visible tokens first .. len-1; wave w takes
    // tiles tbeg + w, tbeg + w + 4, ...
    const int first = window_first(len, window);
    const UnitRun run = split_units(first, len, kTT, split, nsplit);
    const int tbeg = run.begin, tend = run.end;
    const int nmine = tend - tbeg > wave ? (tend - tbeg - wave + kWaves - 1) / kWaves : 0;

    // Q^T operand: column ln = head hg0 + ln, k-chunk = dims 16 s + 8 hh .. +7
    bf16x8 qreg[DS];
    {
        const bool ok = ln < GC;
        const uint16_t* qp = Qp + ((size_t)b * Hq + h0 + (ok ? ln : 0)) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < DS; ++s) qreg[s] = as_bf16x8(ok ? ld16(qp + 16 * s) : make_uint4(0, 0, 0, 0));
    }

    auto vswz = [](int row) { return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); };
    unsigned char* const vs0 = vl0 + wave * VT;       // this wave's V stages
    unsigned char* const vs1 = vl1 + wave * VT;

    // issue tile t (this wave's k-th) into stage st: K into kdst registers,
    // V into LDS. The tile's pages are up to four consecutive table entries,
    // read as scalars (indices clamped to the sequence's last page).
    auto issue = [&](int t, unsigned char* vdst, uint4 (&kdst)[DS], bool dummy) __attribute__((always_inline)) {
        const int j0 = t * kTT;
        const int p0 = j0 >> ps_log2;
        int pid[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pid[i] = __builtin_amdgcn_readfirstlane(tab[min(p0 + i, last_page)]);
        auto pick = [&](int idx) __attribute__((always_inline)) {
            return idx == 0 ? pid[0] : idx == 1 ? pid[1] : idx == 2 ? pid[2] : pid[3];
        };
        // K: lane's token j0 + ln (clamped to len - 1), dims 16 s + 8 hh; a
        // dummy reads the last token's row (valid, and cached after the first)
        const int tok = dummy ? len - 1 : min(j0 + ln, len - 1);
        const int page = dummy ? __builtin_amdgcn_readfirstlane(tab[last_page])
                               : pick(min(max((tok >> ps_log2) - p0, 0), 3));
        const uint16_t* kp = Kp + pool_tile(page, g, Hkv, ps_log2, D) + (size_t)(tok & (ps - 1)) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < DS; ++s) kdst[s] = ld16_nt(kp + 16 * s);
        // V: slot sl holds rows sl * RPS .. +RPS-1, all in one page
#pragma unroll
        for (int sl = 0; sl < VSLOTS; ++sl) {
            const int r0 = j0 + sl * RPS;
            const bool any = !dummy && r0 < len;
            const int vpage = pick(min(max((r0 >> ps_log2) - p0, 0), 3));
            const uint16_t* tile = Vp + pool_tile(vpage, g, Hkv, ps_log2, D);
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)tile, 0, any ? ps * D * 2 : 0, kRsrcWord3);
            const int row = sl * RPS + lane / CPR;
            const int j = j0 + row;
            const int chunk = (lane % CPR) ^ vswz(row);
            const unsigned off = j < len ? (unsigned)((j & (ps - 1)) * D * 2 + 16 * chunk) : (unsigned)(ps * D * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(vdst + sl * 1024), 16, off, 0, 0, 0);
        }
    };

    // V^T operand: a 16-lane group reads 4 tokens x 16 dims transposed
    const int grp = (lane >> 4) & 1;
    const int e4 = (lane & 15) >> 2;
    const int q4 = lane & 3;
    auto vop = [&](const unsigned char* vb, int ks, int db) __attribute__((always_inline)) -> bf16x8 {
        const int key0 = 16 * ks + 4 * hh + e4;
        const int d = 32 * db + 16 * grp + 4 * q4;
        const int o_lo = key0 * (D * 2) + (((d >> 3) ^ vswz(key0)) << 4) + ((d & 7) << 1);
        const int o_hi = o_lo + 8 * (D * 2);     // key0 + 8: same swizzle
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + o_lo));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + o_hi));
        const s16x8 a8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        return __builtin_bit_cast(bf16x8, a8);
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float masked = NEG ? INFINITY : -INFINITY;

    // one tile: logits, mask at the ends of the visible range, online softmax
    // with the lazy reference maximum, O^T += V^T P^T
    auto compute = [&](int t, const uint4 (&kc)[DS], const unsigned char* vb) __attribute__((always_inline)) {
        f32x16 sacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
        for (int s = 0; s < DS; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kc[s]), qreg[s], sacc, 0, 0, 0);
        // accumulator value v holds token j0 + 8 (v / 4) + 4 hh + v % 4 of column ln
        const int j0 = t * kTT;
        if (j0 + kTT > len || j0 < first) {
            asm volatile("");
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = j0 + 8 * (v >> 2) + 4 * hh + (v & 3);
                sacc[v] = (j < len && j >= first) ? sacc[v] : masked;
            }
        }
        float mx = masked;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = NEG ? fminf(mx, sacc[v]) : fmaxf(mx, sacc[v]);
        const float other = __shfl_xor(mx, 32);
        mx = NEG ? fminf(mx, other) : fmaxf(mx, other);
        const float mt = (mx == masked) ? -INFINITY : mx * c2;
        const bool need = mt > m_run + kLazy;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
            m_run = need ? mt : m_run;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        }
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        bf16x8 pb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int jj = 0; jj < 8; jj += 2) {
                const int v0 = 8 * ks + jj;
                f32x2 pr = {__builtin_amdgcn_exp2f(fmaf(sacc[v0], c2, -msub)),
                            __builtin_amdgcn_exp2f(fmaf(sacc[v0 + 1], c2, -msub))};
                const bf16x2 pbf = __builtin_convertvector(pr, bf16x2);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pbf, __builtin_bit_cast(bf16x2, kOnes), l_run, false);
                pb[ks][jj] = pbf[0];
                pb[ks][jj + 1] = pbf[1];
            }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop(vb, ks, db), pb[ks], oacc[db], 0, 0, 0);
    };

    // three register sets for K, rotated with the V stages; tile k of this
    // wave is tile tbeg + wave + 4 k
    uint4 k0[DS], k1[DS];
    issue(tbeg + wave, vs0, k0, nmine <= 0);
    int k = 0;
    auto stage_step = [&](uint4 (&kc)[DS], uint4 (&kn)[DS], const unsigned char* vc, unsigned char* vn)
        __attribute__((always_inline)) {
        // issue tile k + 1 into the stage tile k - 1 used, then tile k
        issue(tbeg + wave + kWaves * (k + 1), vn, kn, k + 1 >= nmine);
        compute(tbeg + wave + kWaves * k, kc, vc);
        ++k;
    };
    while (k < nmine) {
        stage_step(k0, k1, vs0, vs1);
        if (k >= nmine) break;
        stage_step(k1, k0, vs1, vs0);
    }

    // merge the waves: per head column, (m, l) and O^T rows through LDS
    // (the V stages are free once every DMA, dummies included, has landed:
    // waves 0, 1 use stage 0, waves 2, 3 stage 1)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    static_assert(2 * 32 * D * 4 <= kWaves * VT, "merge scratch");
    auto sh_o = [&](int w) __attribute__((always_inline)) {
        return reinterpret_cast<float*>(w < 2 ? vl0 : vl1) + (w & 1) * 32 * D;   // [32 heads][D]
    };
    const float l_tot = l_run + __shfl_xor(l_run, 32);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int d = 32 * db + 8 * (v >> 2) + 4 * hh + (v & 3);
            sh_o(wave)[ln * D + d] = oacc[db][v];
        }
    if (hh == 0) {
        sh_m[wave * 32 + ln] = m_run;
        sh_l[wave * 32 + ln] = l_tot;
    }
    __syncthreads();
    for (int idx = tid; idx < GC * D; idx += kThreads) {
        const int j = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh_m[w * 32 + j]);
        const float M_use = (M == -INFINITY) ? 0.f : M;
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = exp2f(sh_m[w * 32 + j] - M_use);
            L += sh_l[w * 32 + j] * sc;
            acc += sh_o(w)[j * D + d] * sc;
        }
        const size_t unit = ((size_t)b * Hq + h0 + j) * nsplit + split;
        ws[unit * D + d] = acc;
        if (d == 0) {
            float* ml = ws + (size_t)gridDim.z * Hq * nsplit * D;
            ml[2 * unit] = M;
            ml[2 * unit + 1] = L;
        }
    }
}

int heads_per_group(int G) {
    if (G % 8 == 0) return 8;
    if (G % 4 == 0) return 4;
    if (G % 2 == 0) return 2;
    return 1;
}

template <int D, int GH, bool NEG>
void launch_split(const DecodeArgs& a, int ps_log2, float c2, hipStream_t stream) {
    const int groups = a.Hkv * ((a.Hq / a.Hkv) / GH);
    if (log_enabled())
        log_dispatch("decode_split_kernel<%d,%d,%s> B=%d Hq=%d Hkv=%d page_size=%d window=%d: grid %d x %d x %d, "
                     "%d heads per workgroup, %d context splits", D, GH, NEG ? "neg" : "pos", a.B, a.Hq, a.Hkv,
                     a.page_size, a.window, a.nsplit, groups, a.B, GH, a.nsplit);
    hipLaunchKernelGGL((decode_split_kernel<D, GH, NEG>), dim3(a.nsplit, groups, a.B), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_pool, (const uint16_t*)a.v_pool,
                       a.page_table, a.seq_lens, a.ws, a.Hq, a.Hkv, ps_log2, a.nsplit, c2, a.window);
}

template <int D, bool NEG>
void launch_mfma(const DecodeArgs& a, int ps_log2, float c2, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    const int groups = a.Hkv * ((G + 31) / 32);
    // scale 0: a tiny positive factor gives bit-identical weights (every
    // exp2 of a finite logit is 1) and keeps masked logits at -inf instead of
    // -inf * 0 = NaN
    if (c2 == 0.f) c2 = 1e-30f;
    if (log_enabled())
        log_dispatch("decode_mfma_kernel<%d,%s> B=%d Hq=%d Hkv=%d page_size=%d window=%d: grid %d x %d x %d, "
                     "%d context splits", D, NEG ? "neg" : "pos", a.B, a.Hq, a.Hkv, a.page_size, a.window, a.nsplit,
                     groups, a.B, a.nsplit);
    hipLaunchKernelGGL((decode_mfma_kernel<D, NEG>), dim3(a.nsplit, groups, a.B), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_pool, (const uint16_t*)a.v_pool,
                       a.page_table, a.seq_lens, a.ws, a.Hq, a.Hkv, ps_log2, a.nsplit, c2, a.window);
}

template <int D, bool NEG>
void launch_split_d(const DecodeArgs& a, int GH, int ps_log2, float c2, hipStream_t stream) {
    switch (GH) {
        case 8: launch_split<D, 8, NEG>(a, ps_log2, c2, stream); break;
        case 4: launch_split<D, 4, NEG>(a, ps_log2, c2, stream); break;
        case 2: launch_split<D, 2, NEG>(a, ps_log2, c2, stream); break;
        default: launch_split<D, 1, NEG>(a, ps_log2, c2, stream); break;
    }
}

}  // namespace

// Which decode kernel: the vector kernel (three workgroups per CU) is bound
// by its per-byte dot products as the heads per K/V head grow; the MFMA
// kernel (two per CU at D = 128, four at D = 64) has no such cost. Measured
// on MI355X over ten shapes with 8 and more heads per K/V head, the MFMA
// kernel is 6-23 % ahead at D = 128 below 512 (sequence, K/V head) units,
// level at 384 and 3 % behind at 512, up to 1.7x ahead at D = 64 and 1.95x
// at 16 heads; with 4 heads the vector kernel (6 TB/s) is well ahead.
bool decode_on_mfma(int B, int Hq, int Hkv, int D, int num_cu) {
    const int G = Hq / Hkv;
    if (G >= 16) return true;
    if (G < 8) return false;
    return D == 64 || (long long)B * Hkv < 2LL * (num_cu > 0 ? num_cu : 256);
}

int decode_nsplit(int B, int Hq, int Hkv, int num_cu, bool mfma) {
    const int G = Hq / Hkv;
    const long long units = mfma ? (long long)B * Hkv * ((G + 31) / 32)
                                 : (long long)B * Hkv * (G / heads_per_group(G));
    // the MFMA kernel holds fewer workgroups per CU: fewer, longer splits
    // amortise its start (sequence rank, q, the first tile in flight)
    const long long target = (mfma ? 4LL : 8LL) * (num_cu > 0 ? num_cu : 256);
    long long n = (target + units - 1) / units;
    if (n < 1) n = 1;
    if (n > 64) n = 64;
    return (int)n;
}

size_t decode_workspace_floats(int B, int Hq, int D, int nsplit) {
    return (size_t)B * Hq * nsplit * (size_t)(D + 2);
}

hipError_t launch_decode_paged(const DecodeArgs& a, hipStream_t stream) {
    int ps_log2 = 0;
    while ((1 << ps_log2) < a.page_size) ++ps_log2;
    const float c2 = a.scale * 1.4426950408889634f;
    const int GH = heads_per_group(a.Hq / a.Hkv);
    const bool neg = a.scale < 0.f;
    if (a.mfma) {
        if (a.D == 128) {
            if (neg) launch_mfma<128, true>(a, ps_log2, c2, stream);
            else launch_mfma<128, false>(a, ps_log2, c2, stream);
        } else {
            if (neg) launch_mfma<64, true>(a, ps_log2, c2, stream);
            else launch_mfma<64, false>(a, ps_log2, c2, stream);
        }
    } else if (a.D == 128) {
        if (neg) launch_split_d<128, true>(a, GH, ps_log2, c2, stream);
        else launch_split_d<128, false>(a, GH, ps_log2, c2, stream);
    } else {
        if (neg) launch_split_d<64, true>(a, GH, ps_log2, c2, stream);
        else launch_split_d<64, false>(a, GH, ps_log2, c2, stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (log_enabled())
        log_dispatch("decode_merge_kernel<%d>: grid %d x %d threads, %d partials per head", a.D, a.B * a.Hq, a.D,
                     a.nsplit);
    if (a.D == 128)
        hipLaunchKernelGGL((decode_merge_kernel<128>), dim3(a.B * a.Hq), dim3(128), 0, stream,
                           (const float*)a.ws, (uint16_t*)a.o, a.B, a.Hq, a.nsplit);
    else
        hipLaunchKernelGGL((decode_merge_kernel<64>), dim3(a.B * a.Hq), dim3(64), 0, stream,
                           (const float*)a.ws, (uint16_t*)a.o, a.B, a.Hq, a.nsplit);
    return hipGetLastError();
}

}  // namespace attn
