// Attention backward pass, bfloat16 in/out, on gfx950 MFMA.
//
// What it computes: for O = softmax(mask(Q K^T * scale)) V per (batch, query
// head) and an upstream gradient dO, the gradients dQ, dK, dV of
// L = sum(dO * O). With P the softmax weights and S the scaled logits:
// dV = P^T dO, dP = dO V^T, dS = P * (dP - Delta) with
// Delta_i = sum_j P_ij dP_ij = dO_i . O_i, dQ = scale * dS K and
// dK = scale * dS^T Q; a K/V head collects the sums over the query heads that
// read it (GQA, "Attention 机制详解：从 Self-Attention 到 Multi-Query
// Attention" §5.2). P is not stored by the forward pass: it is recomputed
// tile by tile from Q, K and the forward's per-row log-sum-exp, the
// recomputation that the FlashAttention sections of "Attention From Scratch"
// (进阶篇 §5) and "LLM 核心技术：Attention 机制的实现与优化" name as the
// backward half of the method; P = exp2(S * c2 - lse * log2(e)) with
// c2 = scale * log2(e).
//
// Two kernels run in order on the caller's stream:
//  * bwd_dq_kernel, one workgroup per (batch, query head, 128 query rows),
//    four waves of 32 rows. It forms Delta and lse * log2(e) for its rows
//    (stored for the second kernel), keeps its Q and dO rows in registers,
//    then streams 64-key tiles
//    of K and V through LDS as the forward pass does: S^T = K Q^T and
//    dP^T = V dO^T on MFMA (a lane owns one query), then dS, then
//    dQ^T += K^T dS^T with the K^T operand read by the transposing LDS read.
//  * bwd_dkdv_kernel, one workgroup per (batch, kv head, 128 keys) (under a
//    causal mask, per pair of such key blocks), four
//    waves of 32 keys (a lane owns one key), two workgroups per CU whose
//    barriers do not couple, so the two waves of a SIMD drift out of phase
//    and one's softmax runs beside the other's MFMAs. K rows stay in registers and the
//    workgroup's V rows in LDS; it streams 32-row steps of Q, dO, lse and
//    Delta for every query head of the group: S = Q K^T and dP = dO V^T
//    (row operands, 16-byte LDS reads), P, dS, then dV^T += dO^T P and
//    dK^T += Q^T dS with the dO^T and Q^T operands read from the same rows by
//    the transposing LDS read. Summing the group's
//    heads inside one workgroup makes dK and dV plain stores, with no atomics.
//
// Both kernels take the 32x32x16 bf16 MFMA. Tiles are staged by buffer->LDS
// DMA (rows past the end of a slice read as zeros through the buffer range
// check), double buffered. 16-byte chunks of a tile row are XOR-swizzled so
// that the MFMA operand reads avoid bank conflicts. Waves skip 32x32 blocks
// with no visible pair; only blocks that straddle a mask boundary or a tail
// evaluate the mask.

#include "launch.h"
#include "deal.h"

#include <cmath>
#include <type_traits>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kNW = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kRows = 32 * kNW;        // query rows (dq) or keys (dkdv) per workgroup
constexpr int kTile = 64;              // rows of a streamed K/V or Q/dO tile
constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint4 ld_global16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

// XOR swizzle of the 16-byte chunks of tile row `row` (row index within a
// tile that starts at a multiple of 16 rows).
//  * Row operand: 16 lanes read rows r .. r+15 at one logical chunk; the
//    swizzle is a bijection on the low row bits, so they hit 16 different
//    16-byte bank groups (D = 128: one row spans all banks; D = 64: two rows
//    do, and the row parity supplies the missing bit).
//  * Transposing read: 16 lanes read rows r0 .. r0+3 (r0 a multiple of 4),
//    two adjacent chunks each; the swizzle sends the four rows' chunk pairs
//    to four different pairs (D = 128: bits 1-2 carry row & 3; D = 64: rows
//    r0, r0+2 share a parity and differ in bit 1).
// Measured on the dQ kernel: a variant that also keeps the two 16-lane
// halves of a transposing read apart (bits 2-3 = row & 3) counts 16x fewer
// bank-conflict cycles but runs about 20 % slower, so this one stays.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8);
    else return (((row >> 1) & 1) << 1) | ((row >> 2) & 1) | (((row >> 3) & 1) << 2);
}

// MFMA row operand: 8 bf16 of tile row `row`, logical chunk `chunk`.
template <int D>
__device__ __forceinline__ bf16x8 row_op(const unsigned char* t, int row, int chunk) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(t + row * (D * 2) + ((chunk ^ swz<D>(row)) << 4)));
}

// MFMA operand of the transposed tile for one 16-row k step starting at tile
// row `row16`, 32-column block `db`: lane (l % 32, half hh) gets column
// 32*db + l % 32 at rows row16 + 4hh + {0..3} and row16 + 8 + 4hh + {0..3},
// the order in which a 32x32 accumulator hands a lane its rows.
template <int D>
__device__ __forceinline__ bf16x8 tr_op(const unsigned char* t, int row16, int db, int lane) {
    const int hh = lane >> 5, grp = (lane >> 4) & 1, e4 = (lane & 15) >> 2, q4 = lane & 3;
    const int r = row16 + 4 * hh + e4;
    const int d = 32 * db + 16 * grp + 4 * q4;
    const int o_lo = r * (D * 2) + (((d >> 3) ^ swz<D>(r)) << 4) + ((d & 7) << 1);
    const int o_hi = (r + 8) * (D * 2) + (((d >> 3) ^ swz<D>(r + 8)) << 4) + ((d & 7) << 1);
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + o_lo));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + o_hi));
    const s16x8 a8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    return __builtin_bit_cast(bf16x8, a8);
}

// Stage rows r_first .. r_first + kTile - 1 of a [rows, D] bf16 slice into
// `dst`, 1 KiB per wave instruction; the LDS side of a DMA is always
// base + 16 * lane, so the swizzle is applied through the source offset.
template <int D>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int r_first, unsigned char* dst, int wave,
                                         int lane) {
    constexpr int CPR = D / 8;                   // 16-byte chunks per row
    constexpr int RPS = 64 / CPR;                // rows per 1 KiB slot
    constexpr int SLOTS = kTile * D * 2 / 1024;
    static_assert(SLOTS % kNW == 0, "DMA slots per wave");
#pragma unroll
    for (int i = 0; i < SLOTS / kNW; ++i) {
        const int sl = wave + kNW * i;
        const int row = sl * RPS + lane / CPR;
        const int chunk = (lane % CPR) ^ swz<D>(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + sl * 1024), 16,
                                                 (unsigned)(((r_first + row) * D + 8 * chunk) * 2), 0, 0, 0);
    }
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    const f32x2 x = {a, b}, y = {c, d};
    uint2 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    r.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
    return r;
}

// Stores a wave's 32 x D bf16 block, given in the 32x32 MFMA accumulator
// layout (lane ln + 32 hh: row ln, d = 32 db + 8 r + 4 hh .. +3 as the word
// w[db][r]), as rows r0 .. r0 + 31 of a [rows, D] slice, skipping rows at or
// past `nrows`. The block passes through the wave's own 32 x D region of LDS,
// 16-byte chunks XOR-swizzled by row, so that each store instruction writes
// 64 / (D / 8) whole rows instead of 16 bytes of each of 32 rows.
template <int D>
__device__ __forceinline__ void store_block(unsigned char* stage, const uint2 (&w)[D / 32][4], uint16_t* out, int r0,
                                            int nrows, int lane) {
    constexpr int CPR = D / 8;   // 16-byte chunks per row
    const int ln = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<uint2*>(stage + ln * (D * 2) + (((4 * db + r) ^ (ln & (CPR - 1))) << 4) + hh * 8) =
                w[db][r];
    wave_lds_fence();
    const int cl = lane % CPR;
#pragma unroll
    for (int i = 0; i < CPR / 2; ++i) {
        const int row = i * (64 / CPR) + lane / CPR;
        const uint4 x = *reinterpret_cast<const uint4*>(stage + row * (D * 2) + ((cl ^ (row & (CPR - 1))) << 4));
        if (r0 + row < nrows) *reinterpret_cast<uint4*>(out + (size_t)(r0 + row) * D + 8 * cl) = x;
    }
    wave_lds_fence();   // the region may be written again by the next block
}

// 8 values of a 32x32 accumulator (k step `c` of its rows) as a bf16 operand
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int c) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const f32x2 p = {x[8 * c + e], x[8 * c + e + 1]};
        const bf16x2 b = __builtin_convertvector(p, bf16x2);
        r[e] = b[0];
        r[e + 1] = b[1];
    }
    return r;
}

// ---------------------------------------------------------------------------
// dQ (and Delta)

template <int D>
__global__ __launch_bounds__(kThreads, 2)
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                   const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
                   float* __restrict__ Delta, float* __restrict__ L2, uint16_t* __restrict__ dQ, int Hq, int Hkv,
                   int Sq, int Sk, float scale, float c2, int causal, int window, int nqt, int nitems, int chunk,
                   int pair) {
    constexpr int BN = kTile, KB = BN / 32, DS = D / 16, DB = D / 32;
    constexpr int TILE_BYTES = BN * D * 2;
    __shared__ __attribute__((aligned(16))) unsigned char k_lds0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds1[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds1[TILE_BYTES];

    // work item: (batch, kv head) major, then query tile from the heaviest
    // causal one down, then the query heads of the group; dealt to the XCDs
    // as the forward kernels deal theirs
    const int w = blockIdx.x;
    const int item = dealt_item(w, chunk, nitems, pair, nqt, Hq / Hkv);
    if (item < 0) return;
    const int G = Hq / Hkv;
    const int hg = item % G;
    const int r1 = item / G;
    const int qt = nqt - 1 - (r1 % nqt);
    const int bg = r1 / nqt;
    const int g = bg % Hkv;
    const int b = bg / Hkv;
    const int h = g * G + hg;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int ln = lane & 31;
    const int hh = lane >> 5;

    const int off = Sk - Sq;  // bottom-right causal alignment
    const int i0 = qt * kRows;
    const int row_end = min(i0 + kRows, Sq);
    const size_t qo_base = ((size_t)b * Hq + h) * (size_t)Sq * D;
    const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)Sk * D;
    const __amdgpu_buffer_rsrc_t krs = rsrc(K + kv_base, Sk * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = rsrc(V + kv_base, Sk * D * 2);

    const int p_first = i0 + off, p_last = row_end - 1 + off;
    const int hi = causal ? min(Sk, p_last + 1) : Sk;
    const int lo = (causal && window > 0) ? max(0, p_first - window + 1) : 0;
    const int t_begin = lo / BN;
    const int t_end = (hi + BN - 1) / BN;

    const int wr0 = i0 + 32 * wave;
    const int wr1 = min(wr0 + 32, Sq) - 1;
    const bool wave_rows = wr0 < Sq;
    const int wp0 = wr0 + off, wp1 = wr1 + off;
    const int w_hi = causal ? min(Sk - 1, wp1) : Sk - 1;
    const int w_lo = (causal && window > 0) ? max(0, wp0 - window + 1) : 0;
    const int w_full_hi = causal ? min(Sk - 1, wp0) : Sk - 1;
    const int w_full_lo = (causal && window > 0) ? max(0, wp1 - window + 1) : 0;

    // this lane's query row: Q and dO as MFMA B operands (8 d per lane per
    // 16-wide step), Delta = dO . O, lse in log2 units
    const int qrow = wr0 + ln;
    const int qpos = qrow + off;
    const bool row_ok = qrow < Sq;
    bf16x8 qreg[DS], doreg[DS];
    float dsum = 0.f;
    {
        const size_t rb = qo_base + (size_t)(row_ok ? qrow : 0) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            const uint4 z = make_uint4(0, 0, 0, 0);
            qreg[s] = as_bf16x8(row_ok ? ld_global16(Q + rb + 16 * s) : z);
            doreg[s] = as_bf16x8(row_ok ? ld_global16(dO + rb + 16 * s) : z);
            const bf16x8 ob = as_bf16x8(row_ok ? ld_global16(O + rb + 16 * s) : z);
#pragma unroll
            for (int e = 0; e < 8; ++e) dsum = fmaf((float)doreg[s][e], (float)ob[e], dsum);
        }
    }

    const float delta = dsum + __shfl_xor(dsum, 32);
    const size_t row_idx = ((size_t)b * Hq + h) * Sq + qrow;
    const float lse2 = row_ok ? LSE[row_idx] * kLog2e : 0.f;
    if (row_ok && hh == 0) {
        Delta[row_idx] = delta;
        L2[row_idx] = lse2;  // lse in log2 units, for the dK/dV kernel
    }

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) dq[db][v] = 0.f;

    auto issue = [&](int t, unsigned char* kd, unsigned char* vd) __attribute__((always_inline)) {
        dma_tile<D>(krs, t * BN, kd, wave, lane);
        dma_tile<D>(vrs, t * BN, vd, wave, lane);
    };

    // one 32-key block of a tile (keys j0 + 32x .. +31 at tile rows 32x ..)
    auto block = [&](const unsigned char* kb, const unsigned char* vb, int j0, int x, bool edge)
        __attribute__((always_inline)) {
        f32x16 s, dp;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            s[v] = 0.f;
            dp[v] = 0.f;
        }
#pragma unroll
        for (int st = 0; st < DS; ++st) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(kb, 32 * x + ln, 2 * st + hh), qreg[st], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(vb, 32 * x + ln, 2 * st + hh), doreg[st], dp, 0,
                                                         0, 0);
        }
        // exponent of P; masked pairs get -inf, so P = 0 and dS = 0 exactly
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = fmaf(s[v], c2, -lse2);
        if (edge) {
            asm volatile("");
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = j0 + 32 * x + 8 * (v >> 2) + 4 * hh + (v & 3);
                bool ok = j < Sk;
                if (causal) ok = ok && j <= qpos;
                if (window > 0) ok = ok && j > qpos - window;
                s[v] = ok ? s[v] : -INFINITY;
            }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = __builtin_amdgcn_exp2f(s[v]) * (dp[v] - delta);
        // dQ^T += K^T dS^T; k step c covers keys 32x + 16c .. +15 of the tile
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8 dsb = pack8(s, c);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_op<D>(kb, 32 * x + 16 * c, db, lane), dsb, dq[db],
                                                                 0, 0, 0);
        }
    };

    auto step = [&](int t, unsigned char* kc, unsigned char* vc, unsigned char* kn, unsigned char* vn)
        __attribute__((always_inline)) {
        if (t + 1 < t_end) issue(t + 1, kn, vn);
        const int j0 = t * BN;
        const bool active = wave_rows && j0 <= w_hi && j0 + BN - 1 >= w_lo;
        if (active) {
#pragma unroll
            for (int x = 0; x < KB; ++x) {
                const int jb = j0 + 32 * x;
                if (jb > w_hi || jb + 31 < w_lo) continue;
                const bool edge = (jb + 31 > w_full_hi) || (jb < w_full_lo);
                block(kc, vc, j0, x, edge);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    if (t_begin < t_end) {
        issue(t_begin, k_lds0, v_lds0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int t = t_begin; t < t_end; t += 2) {
            step(t, k_lds0, v_lds0, k_lds1, v_lds1);
            if (t + 1 < t_end) step(t + 1, k_lds1, v_lds1, k_lds0, v_lds0);
        }
    }

    // dQ through half a K tile buffer (free after the last barrier)
    if (!wave_rows) return;
    uint2 wq[DB][4];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            wq[db][r] = pack4(dq[db][4 * r] * scale, dq[db][4 * r + 1] * scale, dq[db][4 * r + 2] * scale,
                              dq[db][4 * r + 3] * scale);
    store_block<D>(((wave >> 1) == 0 ? k_lds0 : k_lds1) + (wave & 1) * (32 * D * 2), wq, dQ + qo_base, wr0, Sq,
                   lane);
}

// ---------------------------------------------------------------------------
// dK, dV

constexpr int kKvWaves = 4;               // waves per dK/dV workgroup
constexpr int kKvKeys = 32 * kKvWaves;    // keys per dK/dV workgroup
constexpr int kQB = 32;                   // query rows per streamed step

// Stage `ROWS` rows (from r_first) of a [rows, D] bf16 slice, row-swizzled as
// dma_tile does, spread over NW waves.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, int r_first, unsigned char* dst, int wave,
                                         int lane) {
    constexpr int CPR = D / 8, RPS = 64 / CPR, SLOTS = ROWS * D * 2 / 1024;
    static_assert(SLOTS % NW == 0 || SLOTS < NW, "DMA slots per wave");
#pragma unroll
    for (int i = 0; i < (SLOTS + NW - 1) / NW; ++i) {
        const int sl = wave + NW * i;
        if (SLOTS < NW && sl >= SLOTS) break;
        const int row = sl * RPS + lane / CPR;
        const int chunk = (lane % CPR) ^ swz<D>(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + sl * 1024), 16,
                                                 (unsigned)(((r_first + row) * D + 8 * chunk) * 2), 0, 0, 0);
    }
}

// One workgroup per (batch, kv head, 128 keys), four waves of 32 keys. A
// lane owns one key: its K row is the register B operand of S = Q K^T and its
// V row, read from the workgroup's V block in LDS, that of dP = dO V^T. Each
// step streams 32 query rows of one query head: Q and dO rows (row operands
// of S and dP; through the transposing read, the operands of dV^T += dO^T P
// and dK^T += Q^T dS), lse (log2 units) and Delta.
//
// A step covers one query tile of one head, all heads of the group per tile.
// Under a causal mask key block kt sees the query tiles from about its own
// position to the last, so its work falls with kt. There (with no window and
// one run per key block) workgroup pi takes two key blocks: first nkt-1-pi,
// walking its tiles from the last one down, then pi, walking its tiles from
// the first one up. Every workgroup then does the same work (the two
// blocks' tile counts add up to a constant) in a single round, and at every
// moment all workgroups of one (batch, kv head) are on the same tile in each
// phase, the first-phase ones at tile T - tau, the second-phase ones at tile
// tau - c for the same step count tau, so each tile comes from HBM about once
// per phase (the dK/dV kernel fetches 1.5x its algorithmic bytes at the 4k
// shape, 4.4x with one key block per workgroup, whose second round of blocks
// re-read the tiles staggered). Otherwise workgroup w takes key block
// w / (B * Hkv * nsplit), walking its tiles from the last one down. With
// (batch, kv head) = blockIdx % (B * Hkv), one (batch, kv head) stays on one
// XCD when B * Hkv is a multiple of 8.
//
// When the key blocks are too few to fill the chip (MQA, a single sequence),
// each key block's steps are cut into `nsplit` contiguous runs, one workgroup
// each (blockIdx = (key block * nsplit + split) * B * Hkv + (batch, kv head));
// the runs write float32 partial dK (already scaled) and dV to `part`, which
// bwd_kv_reduce_kernel sums in split order into the bf16 outputs. With one
// run the kernel writes dK and dV itself.
template <int D>
__global__ __launch_bounds__(64 * kKvWaves, 2)
void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ L2, const float* __restrict__ Delta, uint16_t* __restrict__ dK,
                     uint16_t* __restrict__ dV, int Hq, int Hkv, int Sq, int Sk, float scale, float c2, int causal,
                     int window, int nbg, int nsplit, float* __restrict__ part, int nkt, int paired) {
    constexpr int NW = kKvWaves, DS = D / 16, DB = D / 32, NP = 2 * DB;
    constexpr int RT = kQB * D * 2;   // bytes of a row tile
    __shared__ __attribute__((aligned(16))) unsigned char v_lds[kKvKeys * D * 2];
    __shared__ __attribute__((aligned(16))) unsigned char q_lds0[RT];
    __shared__ __attribute__((aligned(16))) unsigned char q_lds1[RT];
    __shared__ __attribute__((aligned(16))) unsigned char o_lds0[RT];    // dO rows
    __shared__ __attribute__((aligned(16))) unsigned char o_lds1[RT];
    __shared__ __attribute__((aligned(16))) float l_lds0[64];            // lse, log2 units (32 used)
    __shared__ __attribute__((aligned(16))) float l_lds1[64];
    __shared__ __attribute__((aligned(16))) float d_lds0[64];            // Delta
    __shared__ __attribute__((aligned(16))) float d_lds1[64];

    const int w = blockIdx.x;
    const int split = paired ? 0 : (w / nbg) % nsplit;
    const int bg = w % nbg;
    // paired: key block nkt - 1 - pi walking the query tiles top-down, then
    // key block pi walking them bottom-up (one block for the middle of an
    // odd count)
    const int pi = w / nbg;
    const int kt_first = paired ? nkt - 1 - pi : w / (nbg * nsplit);
    const int nblk = paired && pi != nkt - 1 - pi ? 2 : 1;
    const int G = Hq / Hkv;
    const int g = bg % Hkv;
    const int b = bg / Hkv;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int ln = lane & 31;
    const int hh = lane >> 5;

    const int off = Sk - Sq;
    auto run_block = [&](int kt, bool down) __attribute__((always_inline)) {
        const int k0 = kt * kKvKeys;
        const int kw0 = k0 + 32 * wave;                 // first key of this wave
        const int kw1 = min(kw0 + 31, Sk - 1);
        const bool wave_keys = kw0 < Sk;
        const int key = kw0 + ln;
        const bool key_ok = key < Sk;

        const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)Sk * D;
        bf16x8 kreg[DS];
        {
            const size_t rb = kv_base + (size_t)(key_ok ? key : 0) * D + 8 * hh;
#pragma unroll
            for (int s = 0; s < DS; ++s)
                kreg[s] = as_bf16x8(key_ok ? ld_global16(K + rb + 16 * s) : make_uint4(0, 0, 0, 0));
        }

        // queries that see at least one key of the workgroup: position p = q + off
        // sees key j iff j <= p (causal) and j > p - window
        const int kmax = min(k0 + kKvKeys, Sk) - 1;
        const int q_lo = causal ? max(0, k0 - off) : 0;
        const int q_hi = (causal && window > 0) ? min(Sq - 1, kmax + window - 1 - off) : Sq - 1;
        const int t_hi = q_hi / kQB;
        const int t_lo = q_lo / kQB;
        const int nt = q_lo <= q_hi ? t_hi - t_lo + 1 : 0;
        // query tile of step s
        auto tile_of = [&](int s) __attribute__((always_inline)) { return down ? t_hi - s / G : t_lo + s / G; };
        const int nsteps = G * nt;
        // this workgroup's run of steps
        const int s_begin = (int)((long long)nsteps * split / nsplit);
        const int s_end = (int)((long long)nsteps * (split + 1) / nsplit);

        f32x16 dk[DB], dv[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                dk[db][v] = 0.f;
                dv[db][v] = 0.f;
            }

        // step s: query tile t_hi - s / G of query head g * G + s % G
        auto issue = [&](int s, unsigned char* qd, unsigned char* od, float* ld, float* dd)
            __attribute__((always_inline)) {
            const int t = tile_of(s);
            const int bh = b * Hq + g * G + s % G;
            const size_t rows = (size_t)bh * Sq;
            dma_rows<D, kQB, NW>(rsrc(Q + rows * D, Sq * D * 2), t * kQB, qd, wave, lane);
            dma_rows<D, kQB, NW>(rsrc(dO + rows * D, Sq * D * 2), t * kQB, od, wave, lane);
            if (wave == NW - 1)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(L2 + rows, Sq * 4), (lds_void*)ld, 4,
                                                         (unsigned)((t * kQB + lane) * 4), 0, 0, 0);
            else if (wave == NW - 2)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(Delta + rows, Sq * 4), (lds_void*)dd, 4,
                                                         (unsigned)((t * kQB + lane) * 4), 0, 0, 0);
        };
        // does step s have a visible (query, key) pair for this wave; does it
        // need the mask (a boundary or a tail crosses it)
        auto visible_step = [&](int s, bool& edge) __attribute__((always_inline)) {
            const int qa = tile_of(s) * kQB;
            const int pa = qa + off, pe = min(qa + kQB - 1, Sq - 1) + off;
            const bool any = wave_keys && (!causal || kw0 <= pe) && (window == 0 || kw1 > pa - window);
            edge = !((qa + kQB - 1 < Sq) && (kw0 + 31 < Sk) && (!causal || kw0 + 31 <= pa) &&
                     (window == 0 || kw0 > pe - window));
            return any;
        };

        // LDS addresses: with 2st + hh = 2st ^ hh, chunk (2st + hh) ^ sw of a row
        // is chunk hh ^ sw XOR 2st, so the byte offset of k step st is a per-lane
        // base XOR (st << 5) and a tile's base is the instruction's immediate
        // offset. The bases are made opaque at each use so the compiler recomputes
        // the XORs instead of keeping one address register per k step.
        const int sw = swz<D>(ln) ^ hh;
        auto ld16 = [](const unsigned char* p) __attribute__((always_inline)) {
            return as_bf16x8(*reinterpret_cast<const uint4*>(p));
        };

        // S and dP of one step, then P and dS packed as bf16 operands. Operands
        // are read one k step ahead of their MFMAs, and the scheduling barriers
        // keep the compiler from hoisting more reads than that (the register file
        // holds K, dK and dV for the whole kernel).
        auto forward_part = [&](const unsigned char* qb, const unsigned char* ob, const float* lb, const float* dlb,
                                int qa, bool edge, bf16x8* pb, bf16x8* dsb) __attribute__((always_inline)) {
            int aq = ln * (D * 2) + (sw << 4);
            int av = (32 * wave + ln) * (D * 2) + (sw << 4);
            asm volatile("" : "+v"(aq), "+v"(av));
            f32x16 S, P;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                S[v] = 0.f;
                P[v] = 0.f;
            }
            bf16x8 aqo = ld16(qb + aq), aoo = ld16(ob + aq), avo = ld16(v_lds + av);
            // the two waves of a SIMD meet at every barrier and would run their
            // MFMA and softmax phases side by side; a raised priority while a wave
            // issues MFMAs lets the first one through its block, so the other's
            // VALU work overlaps it (about 1.5 % on the dK/dV kernel; in the dQ
            // kernel, two workgroups per CU and no such lockstep, it costs 2 %)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int st = 0; st < DS; ++st) {
                bf16x8 nq = aqo, no = aoo, nv = avo;
                if (st + 1 < DS) {
                    const int x = (st + 1) << 5;
                    nq = ld16(qb + (aq ^ x));
                    no = ld16(ob + (aq ^ x));
                    nv = ld16(v_lds + (av ^ x));
                }
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aqo, kreg[st], S, 0, 0, 0);
                P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aoo, avo, P, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                aqo = nq;
                aoo = no;
                avo = nv;
            }
            __builtin_amdgcn_s_setprio(0);
            // accumulator value v holds query row 8(v/4) + 4hh + v%4 of the step;
            // masked pairs get an exponent of -inf, so P = 0 and dS = 0 exactly
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 l4 = *reinterpret_cast<const float4*>(lb + 8 * j + 4 * hh);
                const float l[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) S[4 * j + i] = fmaf(S[4 * j + i], c2, -l[i]);
            }
            if (edge) {
                asm volatile("");
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int q = qa + 8 * (v >> 2) + 4 * hh + (v & 3);
                    const int p = q + off;
                    bool ok = q < Sq && key_ok;
                    if (causal) ok = ok && key <= p;
                    if (window > 0) ok = ok && key > p - window;
                    S[v] = ok ? S[v] : -INFINITY;
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 d4 = *reinterpret_cast<const float4*>(dlb + 8 * j + 4 * hh);
                const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = 4 * j + i;
                    S[v] = __builtin_amdgcn_exp2f(S[v]);
                    P[v] = S[v] * (P[v] - dl[i]);
                }
            }
            pb[0] = pack8(S, 0);
            pb[1] = pack8(S, 1);
            dsb[0] = pack8(P, 0);
            dsb[1] = pack8(P, 1);
            __builtin_amdgcn_sched_barrier(0);
        };

        // dV^T += dO^T P, dK^T += Q^T dS; k step c covers the step's rows
        // 16c .. 16c+15; operands one (c, d) pair ahead
        auto backward_part = [&](const bf16x8* pb, const bf16x8* dsb, const unsigned char* qb, const unsigned char* ob)
            __attribute__((always_inline)) {
            bf16x8 to = tr_op<D>(ob, 0, 0, lane), tq = tr_op<D>(qb, 0, 0, lane);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int x = 0; x < NP; ++x) {
                const int c = x / DB, d = x % DB;
                bf16x8 no = to, nq = tq;
                if (x + 1 < NP) {
                    no = tr_op<D>(ob, 16 * ((x + 1) / DB), (x + 1) % DB, lane);
                    nq = tr_op<D>(qb, 16 * ((x + 1) / DB), (x + 1) % DB, lane);
                }
                dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(to, pb[c], dv[d], 0, 0, 0);
                dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq, dsb[c], dk[d], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                to = no;
                tq = nq;
            }
            __builtin_amdgcn_s_setprio(0);
        };

        // step s, its tiles in the buffers of parity R (compile-time, so that
        // every LDS address is a constant offset)
        auto step = [&](int s, auto r2) __attribute__((always_inline)) {
            constexpr int R = decltype(r2)::value;
            if (s + 1 < s_end)
                issue(s + 1, R ? q_lds0 : q_lds1, R ? o_lds0 : o_lds1, R ? l_lds0 : l_lds1, R ? d_lds0 : d_lds1);
            bool edge;
            if (visible_step(s, edge)) {
                bf16x8 pb[2], dsb[2];
                forward_part(R ? q_lds1 : q_lds0, R ? o_lds1 : o_lds0, R ? l_lds1 : l_lds0, R ? d_lds1 : d_lds0,
                             tile_of(s) * kQB, edge, pb, dsb);
                backward_part(pb, dsb, R ? q_lds1 : q_lds0, R ? o_lds1 : o_lds0);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };

        if (s_end > s_begin) {
            // the workgroup's V rows stay in LDS for the whole kernel
            dma_rows<D, kKvKeys, NW>(rsrc(V + kv_base, Sk * D * 2), k0, v_lds, wave, lane);
            issue(s_begin, q_lds0, o_lds0, l_lds0, d_lds0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            for (int s = s_begin; s < s_end; s += 2) {
                step(s, std::integral_constant<int, 0>());
                if (s + 1 < s_end) step(s + 1, std::integral_constant<int, 1>());
            }
        }

        // accumulator value v of block db holds d = 32 db + 8(v/4) + 4hh + v%4
        if (!wave_keys) return;
        if (part != nullptr) {
            const size_t plane = (size_t)nbg * Sk * D;
            if constexpr (D == 128) {
                // float partials, 64 columns (two d blocks, 256 bytes of a row)
                // per pass through the wave's 8 KiB of V rows in LDS, read back
                // as whole 256-byte row segments, four rows per store instruction
                unsigned char* stage = v_lds + wave * (32 * D * 2);
                const int cl = lane & 15;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    float* base = part + (size_t)(m * nsplit + split) * plane + ((size_t)bg * Sk + kw0) * D;
#pragma unroll
                    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                        for (int x = 0; x < 2; ++x)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const f32x16& acc = m == 0 ? dk[2 * pass + x] : dv[2 * pass + x];
                                const float s = m == 0 ? scale : 1.f;
                                const int chunk = (8 * x + 2 * r + hh) ^ (ln & 15);
                                *reinterpret_cast<float4*>(stage + ln * 256 + chunk * 16) =
                                    make_float4(acc[4 * r] * s, acc[4 * r + 1] * s, acc[4 * r + 2] * s,
                                                acc[4 * r + 3] * s);
                            }
                        wave_lds_fence();
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int row = 4 * i + (lane >> 4);
                            const float4 v4 =
                                *reinterpret_cast<const float4*>(stage + row * 256 + ((cl ^ (row & 15)) << 4));
                            if (kw0 + row < Sk)
                                *reinterpret_cast<float4*>(base + (size_t)row * D + 64 * pass + 4 * cl) = v4;
                        }
                        wave_lds_fence();   // the next pass writes the same region
                    }
                }
                return;
            }
            if (!key_ok) return;
            float* kp = part + (size_t)split * plane + ((size_t)bg * Sk + key) * D;
            float* vp = part + (size_t)(nsplit + split) * plane + ((size_t)bg * Sk + key) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 32 * db + 8 * r + 4 * hh;
                    *reinterpret_cast<float4*>(kp + d) =
                        make_float4(dk[db][4 * r] * scale, dk[db][4 * r + 1] * scale, dk[db][4 * r + 2] * scale,
                                    dk[db][4 * r + 3] * scale);
                    *reinterpret_cast<float4*>(vp + d) =
                        make_float4(dv[db][4 * r], dv[db][4 * r + 1], dv[db][4 * r + 2], dv[db][4 * r + 3]);
                }
            return;
        }
        // dK, then dV, through the wave's own V rows in LDS (no longer needed)
        uint2 wk[DB][4], wv[DB][4];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wk[db][r] = pack4(dk[db][4 * r] * scale, dk[db][4 * r + 1] * scale, dk[db][4 * r + 2] * scale,
                                  dk[db][4 * r + 3] * scale);
                wv[db][r] = pack4(dv[db][4 * r], dv[db][4 * r + 1], dv[db][4 * r + 2], dv[db][4 * r + 3]);
            }
        unsigned char* stage = v_lds + wave * (32 * D * 2);
        store_block<D>(stage, wk, dK + kv_base, kw0, Sk, lane);
        store_block<D>(stage, wv, dV + kv_base, kw0, Sk, lane);
    };
    run_block(kt_first, true);
    if (nblk == 2) {
        __syncthreads();   // the V rows and the staging area are reused
        run_block(pi, false);
    }
}

// dK, dV of a split key block: the sum, in split order, of the runs' float32
// partials (four elements per thread), rounded to bf16
__global__ __launch_bounds__(256)
void bwd_kv_reduce_kernel(const float* __restrict__ part, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                          long long plane, int nsplit) {
    const long long i = 4 * ((long long)blockIdx.x * 256 + threadIdx.x);
    if (i >= plane) return;
    float4 k = make_float4(0.f, 0.f, 0.f, 0.f), v = k;
    for (int z = 0; z < nsplit; ++z) {
        const float4 a = *reinterpret_cast<const float4*>(part + (size_t)z * plane + i);
        const float4 c = *reinterpret_cast<const float4*>(part + (size_t)(nsplit + z) * plane + i);
        k.x += a.x; k.y += a.y; k.z += a.z; k.w += a.w;
        v.x += c.x; v.y += c.y; v.z += c.z; v.w += c.w;
    }
    *reinterpret_cast<uint2*>(dK + i) = pack4(k.x, k.y, k.z, k.w);
    *reinterpret_cast<uint2*>(dV + i) = pack4(v.x, v.y, v.z, v.w);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int D>
hipError_t launch_d(const BackwardArgs& a, hipStream_t stream) {
    const float c2 = a.scale * kLog2e;
    // workspace: Delta and lse in log2 units, each [B, Hq, Sq] float32, then
    // the split partials of dK and dV (several runs per key block only)
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    const size_t rbytes = align256((size_t)a.B * a.Hq * a.Sq * 4);
    float* delta = reinterpret_cast<float*>(ws);
    float* l2 = reinterpret_cast<float*>(ws + rbytes);
    if (a.Sq > 0) {
        const int nqt = (a.Sq + kRows - 1) / kRows;
        const long long nitems = (long long)a.B * a.Hq * nqt;
        const int G = a.Hq / a.Hkv;
        const Deal deal = make_deal(nitems, (long long)G * nqt, G, false);
        const long long grid = deal.grid;
        // causal items: order by weight (two workgroups per CU)
        const int pair = balance_arg(nitems, deal.chunk, (long long)G * nqt, grid, a.causal, a.num_cu, 2);
        if (!grid_fits(grid, kThreads)) return hipErrorInvalidValue;
        if (log_enabled())
            log_dispatch("bwd_dq_kernel<%d> B=%d Hq=%d Hkv=%d Sq=%d Sk=%d causal=%d window=%d: grid %lld x %d "
                         "threads, %lld items of %d rows, chunk %lld, balance %d", D, a.B, a.Hq, a.Hkv, a.Sq, a.Sk,
                         a.causal, a.window, grid, kThreads, nitems, kRows, deal.chunk, pair);
        hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.o,
                           (const uint16_t*)a.dout, a.lse, delta, l2, (uint16_t*)a.dq, a.Hq, a.Hkv, a.Sq, a.Sk,
                           a.scale, c2, a.causal, a.window, nqt, (int)nitems, (int)deal.chunk, pair);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nkt = (a.Sk + kKvKeys - 1) / kKvKeys;
    const int nbg = a.B * a.Hkv;
    const int nsplit = a.Sq > 0 ? a.kv_splits : 1;
    float* part = nsplit > 1 ? reinterpret_cast<float*>(ws + 2 * rbytes) : nullptr;
    // causal, no window, one run per key block: key blocks in pairs (the
    // light one first, top-down; the heavy one second, bottom-up), one round
    // of equal work
    const int paired = nsplit == 1 && a.causal && a.window == 0 && nkt >= 2 ? 1 : 0;
    const long long grid = paired ? (long long)nbg * ((nkt + 1) / 2) : (long long)nbg * nkt * nsplit;
    if (!grid_fits(grid, 64 * kKvWaves)) return hipErrorInvalidValue;
    if (log_enabled())
        log_dispatch("bwd_dkdv_kernel<%d>: grid %lld x %d threads, %d key blocks of %d per (batch, kv head)%s, "
                     "%d query splits%s", D, grid, 64 * kKvWaves, nkt, kKvKeys, paired ? " in pairs" : "", nsplit,
                     nsplit > 1 ? " + bwd_kv_reduce_kernel" : "");
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)grid), dim3(64 * kKvWaves), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                       l2, delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.Hq, a.Hkv, a.Sq, a.Sk, a.scale, c2,
                       a.causal, a.window, nbg, nsplit, part, nkt, paired);
    if (nsplit > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const long long plane = (long long)nbg * a.Sk * D;
        const long long blocks = (plane / 4 + 255) / 256;
        hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const float*)part,
                           (uint16_t*)a.dk, (uint16_t*)a.dv, plane, nsplit);
    }
    return hipGetLastError();
}

}  // namespace

int backward_kv_splits(int B, int Hkv, int Sq, int Sk, int num_cu) {
    // enough dK/dV workgroups for two per CU, at most 16 runs per key block
    if (Sq <= 0) return 1;
    const long long units = (long long)B * Hkv * ((Sk + kKvKeys - 1) / kKvKeys);
    const long long target = 2LL * (num_cu > 0 ? num_cu : 256);
    long long n = units > 0 ? (target + units - 1) / units : 1;
    if (n < 1) n = 1;
    if (n > 16) n = 16;
    return (int)n;
}

size_t backward_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kv_splits) {
    (void)D;
    size_t bytes = 2 * align256((size_t)B * Hq * Sq * 4);
    if (kv_splits > 1) bytes += 2 * (size_t)kv_splits * B * Hkv * Sk * D * 4;
    return bytes;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
    return a.D == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace attn
