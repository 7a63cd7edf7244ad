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
// One kernel, prefill_pipe_kernel (software pipelined, described above its
// definition), for D = 128 (eight waves and 256 query rows per workgroup, or
// four waves and 128 rows) and D = 64 (four waves and 128 rows, three
// workgroups per CU). The gfx950 mapping:
//  * 32 query rows per wave. Each wave computes S^T = K_tile · Q^T with
//    v_mfma_f32_32x32x16_bf16, so a lane owns one query column and 16 key
//    rows of each 32-key block; the row maximum of a query is a reduction
//    over the lane's own values plus one exchange with lane ^ 32.
//  * Q lives in registers for the whole loop (it is the MFMA B operand).
//  * K and V tiles are staged through LDS by buffer->LDS DMA, double
//    buffered. 16-byte chunks are XOR-swizzled by row so the MFMA operand
//    reads (32 rows at one column) hit distinct banks.
//  * O^T = V^T · P^T also runs on MFMA; P^T comes straight from the S^T
//    accumulators (converted to bf16 in registers); the V^T operand is read
//    from V in its natural layout with the transposing LDS read.
//  * Tiles wholly outside a wave's causal/window range are skipped; only
//    tiles that straddle a boundary or the key tail evaluate the mask.
//  * Work items are ordered (batch, kv head) major, then query tile from the
//    heaviest causal tile down, then the query heads of the group. The item
//    list is cut into chunks that are dealt to the XCDs in snake order
//    (0..7, 7..0, ...) and each XCD runs its chunks in list order, so the
//    query heads sharing a K/V head meet in the same L2. Contiguous K/V uses
//    one chunk per XCD; a paged cache, whose sequences differ in length and
//    are listed longest first, uses one (batch, kv head) group per chunk, so
//    every XCD gets a like share of long and short sequences. With fewer
//    groups than XCDs (MQA, one sequence) a chunk is one query tile's heads,
//    so every XCD gets a like share of heavy and light causal tiles. With
//    causal contiguous K/V and a single round of workgroups, or groups too
//    small to fill two rounds of an XCD, each XCD takes its items heaviest
//    query tile first across its groups (deal.h).

#include "launch.h"
#include "deal.h"
#include "paging.h"

#include <algorithm>
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint4 ld_global16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;
// Lazy-rescale threshold for the reference maximum, log2 units.
constexpr float kLazy = 8.0f;

// ---------------------------------------------------------------------------
// Software pipelined. Per wave and K/V tile t, one basic block holds
//  * an S phase of eight chunks: D/64 MFMAs per chunk of S(t+1) = K(t+1)·Q^T
//    (their K operands read from LDS a chunk ahead) beside the exp2 / bf16
//    conversion of one eighth of P(t), so the matrix and vector units work at
//    the same time;
//  * a P·V phase (chunks 2-9): D/64 MFMAs per chunk of O^T += V(t)^T·P(t)^T
//    (the transposing V reads one chunk ahead) beside the row maximum of
//    S(t+1); the mask of a boundary tile and the lazy move of the reference
//    maximum for tile t+1 follow the block.
// The O rescale that a moved maximum asks for runs at the start of the next
// step, in a branch taken only when some lane of the wave needs it.
// sched_barrier fences keep the chunks in this order; inside a chunk the
// compiler interleaves freely. S(t+1) is accumulated 32-key block 1 first,
// block 0 second, while P(t) consumes block 0 first: only three of the four
// 16-register blocks of S(t) and S(t+1) are live at any time.
// K is staged one tile ahead of V: during step t the LDS holds K(t+1) and
// V(t) while the DMA fills K(t+2) and V(t+1); the step's DMA goes out after
// chunk 1 of the block rather than right after the barrier, where every wave
// of the CU would issue its share at the same moment.

__device__ __forceinline__ float2 halves(float x) {
    // lanes l and l ^ 32 of x, in every lane (v_permlane32_swap)
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x), false, false);
    return make_float2(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// PAGED: K and V come from a paged cache ([pages, Hkv, ps, D] pools, a
// ragged page table and per-sequence lengths, the layout of the paged decode)
// instead of [B, Hkv, Sk, D] slices; Sk is then the sequence's length.
template <int NW, int D, bool NEG, bool PAGED>
__global__ __launch_bounds__(64 * NW, D == 64 ? 3 : 2)
void prefill_pipe_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                         const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                         int Hq, int Hkv, int Sq, int Sk, float c2, int causal, int window,
                         int nqt, int nitems, int chunk, int pair,
                         const int32_t* __restrict__ table, const int32_t* __restrict__ lens, int ps_log2) {
    static_assert(D == 64 || D == 128, "head dimension");
    constexpr int BN = 64, KB = 2, KS = 4, DS = D / 16, DB = D / 32, CPR = D / 8;
    constexpr int RPS = 1024 / (D * 2);   // K/V rows per 1 KiB DMA slot
    constexpr int SPC = DS / 4;           // S-steps of S(t+1) per chunk and block
    constexpr int DPC = DB / 2;           // d blocks of O per P·V chunk
    constexpr int TILE_BYTES = BN * D * 2;
    constexpr int SLOTS = TILE_BYTES / 1024;
    constexpr int BMW = 32 * NW;  // query rows per workgroup
    static_assert(SLOTS % NW == 0, "DMA slots per wave");

    __shared__ __attribute__((aligned(16))) unsigned char k_lds0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char k_lds1[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds0[TILE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char v_lds1[TILE_BYTES];

    const int w = blockIdx.x;
    const int item = dealt_item(w, chunk, nitems, pair, nqt, Hq / Hkv);
    if (item < 0) return;
    const int G = Hq / Hkv;
    const int hg = item % G;
    const int r1 = item / G;
    const int qt = nqt - 1 - (r1 % nqt);
    const int bg = r1 / nqt;
    const int g = bg % Hkv;
    int b = bg / Hkv;
    const int h = g * G + hg;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int ln = lane & 31;
    const int hh = lane >> 5;

    // paged: the sequence's length and its first page-table entry
    // off_b = sum over j < b of ceil(lens[j] / page_size)
    int off_b = 0;
    if constexpr (PAGED) {
        // sequence slot b of the grid takes the sequence of b-th largest length
        // (ties by index; up to 64 * NW sequences), so the longest caches,
        // the most work, are dispatched first
        const int B = nitems / (Hq * nqt);
        if (B <= 64 * NW) {
            __shared__ int sh_seq;
            if (tid < B) {
                const int my = lens[tid];
                int rank = 0;
                for (int j = 0; j < B; ++j) {
                    const int lj = lens[j];
                    rank += (lj > my) || (lj == my && j < tid);
                }
                if (rank == b) sh_seq = tid;
            }
            __syncthreads();
            b = sh_seq;
        }
        __shared__ int sh_part[NW];
        int part = 0;
        for (int j = tid; j < b; j += 64 * NW) part += seq_pages(lens[j], ps_log2);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
        if (lane == 0) sh_part[wave] = part;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < NW; ++x) off_b += sh_part[x];
        Sk = lens[b];
        if (Sk < 1) return;   // outside the precondition seq_lens[b] >= 1: nothing to do
    }

    const int off = Sk - Sq;
    const int i0 = qt * BMW;
    const int row_end = min(i0 + BMW, Sq);

    const size_t qo_base = ((size_t)b * Hq + h) * (size_t)Sq * D;
    const size_t kv_base = PAGED ? 0 : ((size_t)b * Hkv + g) * (size_t)Sk * D;
    const int kv_bytes = PAGED ? 0 : Sk * D * 2;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(K + kv_base), 0, kv_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(V + kv_base), 0, kv_bytes, kRsrcWord3);

    const int p_first = i0 + off;
    const int p_last = row_end - 1 + off;
    const int hi = causal ? min(Sk, p_last + 1) : Sk;
    const int lo = (causal && window > 0) ? max(0, p_first - window + 1) : 0;
    const int t_begin = lo / BN;
    const int t_end = (hi + BN - 1) / BN;

    // Rows of this wave. With eight waves the 32-row blocks are dealt so that
    // the two waves sharing a SIMD (w and w + 4) hold one early and one late
    // block: under a causal mask their tile counts then add up to the same
    // total on every SIMD.
    const int blk = (NW == 8 && wave >= 4) ? 11 - wave : wave;
    const int wr0 = i0 + 32 * blk;
    const int wr1 = min(wr0 + 32, Sq) - 1;
    const int wp0 = wr0 + off, wp1 = wr1 + off;
    // tiles wholly visible to all rows of the wave need no mask
    const int w_full_hi = causal ? min(Sk - 1, wp0) : Sk - 1;
    const int w_full_lo = (causal && window > 0) ? max(0, wp1 - window + 1) : 0;
    // last tile with a key visible to the wave (before t_begin: no rows)
    const int wt_hi = wr0 >= Sq ? t_begin - 1 : (causal ? min(Sk - 1, wp1) / BN : t_end - 1);
    auto is_edge = [&](int t) __attribute__((always_inline)) { return (t * BN + BN - 1 > w_full_hi) || (t * BN < w_full_lo); };

    const int qrow = wr0 + ln;
    const int qpos = qrow + off;
    bf16x8 qreg[DS];

    // K rows keep their 16-byte chunks XOR-swizzled by kswz(row), V rows by
    // vswz(row) (D = 128: row & 15 and (row & 3) << 2; D = 64, 8 chunks per
    // row: (row >> 1) & 7 and ((row >> 1) & 1) << 2), so the MFMA operand
    // reads of 32 rows at one column and the transposing V reads hit
    // distinct banks; the DMA realises the swizzle through the source offset.
    // 1 KiB per wave instruction holds RPS rows (4 at D = 128, 8 at D = 64);
    // slot i of a wave covers rows RPS (NW i + wave) + lane / CPR, so the
    // swizzle (low row bits) and the lane's byte offset are the same for
    // every slot. The whole offset goes in the VGPR operand, which the buffer
    // range check covers; the row part is made opaque so the compiler adds it
    // per tile instead of keeping one VGPR per slot.
    auto kswz = [](int row) __attribute__((always_inline)) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
    auto vswz = [](int row) __attribute__((always_inline)) {
        return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
    };
    const int dma_row = RPS * wave + lane / CPR;
    static_assert(SLOTS / NW >= 1, "DMA slots");
    const unsigned kv_lane_k = (unsigned)((dma_row * D + 8 * ((lane % CPR) ^ kswz(dma_row))) * 2);
    const unsigned kv_lane_v = (unsigned)((dma_row * D + 8 * ((lane % CPR) ^ vswz(dma_row))) * 2);
    // paged: the RPS rows of a slot start at a multiple of RPS and so lie in
    // one page (page_size >= 8); the slot gets a buffer resource over that
    // (page, kv head) tile, and rows at or past Sk (or a slot wholly past it,
    // whose page is not even looked up) read zeros through the range check
    const int ps = 1 << ps_log2;
    const unsigned pg_lane_k = (unsigned)((8 * ((lane % CPR) ^ kswz(dma_row))) * 2);
    const unsigned pg_lane_v = (unsigned)((8 * ((lane % CPR) ^ vswz(dma_row))) * 2);
    // paged: the page ids of the slots a wave loads in the next step are
    // fetched one step ahead by a vector load (lane i < SPW: K slot i of tile
    // tk; lane SPW + i: V slot i of tile tv) and taken back with readlane. A
    // scalar load right before the DMA would stall the wave, and its wait
    // (the counter scalar loads share with LDS reads) would also wait for
    // the step's first K operand reads.
    constexpr int SPW = SLOTS / NW;
    auto page_ids = [&](int tk, int tv) __attribute__((always_inline)) {
        int id = 0;
        if constexpr (PAGED) {
            if (lane < 2 * SPW) {
                const bool v_slot = lane >= SPW;
                const int i = v_slot ? lane - SPW : lane;
                const int tt = v_slot ? tv : tk;
                const int j0 = tt * BN + RPS * NW * i + RPS * wave;
                if (tt < t_end && j0 < Sk) id = table[off_b + (j0 >> ps_log2)];
            }
        }
        return id;
    };
    auto issue = [&](__amdgpu_buffer_rsrc_t rs, int t, unsigned char* dst, bool is_v, int pid = 0,
                     bool have_pid = false) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SLOTS / NW; ++i) {
            const int sl = wave + NW * i;
            if constexpr (PAGED) {
                const int j0 = t * BN + RPS * NW * i + RPS * wave;     // first row of the slot
                const bool any = j0 < Sk;
                const int page = !any ? 0
                                 : have_pid ? __builtin_amdgcn_readlane(pid, (is_v ? SPW : 0) + i)
                                            : table[off_b + (j0 >> ps_log2)];
                const uint16_t* tile = (is_v ? V : K) + pool_tile(page, g, Hkv, ps_log2, D);
                const __amdgpu_buffer_rsrc_t pr =
                    __builtin_amdgcn_make_buffer_rsrc((void*)tile, 0, any ? ps * D * 2 : 0, kRsrcWord3);
                const int j = j0 + lane / CPR;
                const unsigned voff = j < Sk ? (unsigned)((j & (ps - 1)) * D * 2) + (is_v ? pg_lane_v : pg_lane_k)
                                             : (unsigned)(ps * D * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(pr, (lds_void*)(dst + sl * 1024), 16, voff, 0, 0, 0);
            } else {
                unsigned rows = (unsigned)((t * BN + RPS * NW * i) * D * 2);
#if defined(__HIP_DEVICE_COMPILE__)
                asm volatile("" : "+s"(rows));
#endif
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + sl * 1024), 16,
                                                         (unsigned)((is_v ? kv_lane_v : kv_lane_k) + rows), 0, 0, 0);
            }
        }
    };
    // K operand (A: key = lane % 32) of S-step st, keys 32*kbk .. +31
    auto kread = [&](const unsigned char* kb, int st, int kbk) __attribute__((always_inline)) -> bf16x8 {
        const int key = 32 * kbk + ln;
        const int cc = 2 * st + hh;
        return as_bf16x8(*reinterpret_cast<const uint4*>(kb + key * (D * 2) + ((cc ^ kswz(key)) << 4)));
    };
    // V^T operand of P·V k-step ks, d block db: for k-step ks the S^T
    // accumulators hand lane half hh the keys 16ks + 4hh + {0..3} and
    // 16ks + 8 + 4hh + {0..3}; two transposing reads fetch exactly those
    const int grp = (lane >> 4) & 1;
    const int e4 = (lane & 15) >> 2;
    const int q4 = lane & 3;
    auto vop = [&](const unsigned char* vb, int ks, int db) __attribute__((always_inline)) -> bf16x8 {
        const int key0 = 16 * ks + 4 * hh + e4;
        const int d = 32 * db + 16 * grp + 4 * q4;
        const int o_lo = key0 * (D * 2) + (((d >> 3) ^ vswz(key0)) << 4) + ((d & 7) << 1);
        const int o_hi = o_lo + 8 * (D * 2);  // key0 + 8 has the same swizzle
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
    // Reference maximum of the scaled logits (log2 units), moved only when a
    // tile exceeds it by more than kLazy; numerator and denominator share it.
    float m_run = -INFINITY;
    float l_run = 0.f;
    float alpha = 1.f;      // O rescale owed for the next tile
    bool rescale = false;   // wave-uniform: some lane owes one
    const uint32_t ones = 0x3F803F80u;
    const float masked = NEG ? INFINITY : -INFINITY;

    // mask of the 8 S values of block kbk, elements 8*half .. +7 (edge tiles)
    auto mask8 = [&](f32x16& sb, int j0, int kbk, int half) __attribute__((always_inline)) {
        const int base = j0 + 4 * hh;
        const int sk_hi = Sk - 1 - base;
        const int lim_hi = causal ? min(qpos - base, sk_hi) : sk_hi;
        const int lim_lo = window > 0 ? qpos - window - base : -1;
#pragma unroll
        for (int v = 8 * half; v < 8 * half + 8; ++v) {
            const int c = 32 * kbk + 8 * (v >> 2) + (v & 3);
            const bool ok = c <= lim_hi && c > lim_lo;
            sb[v] = ok ? sb[v] : masked;
        }
    };
    auto ext8 = [&](const f32x16& sb, int half, float mx) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 8 * half; v < 8 * half + 8; ++v) mx = NEG ? fminf(mx, sb[v]) : fmaxf(mx, sb[v]);
        return mx;
    };
    // the extreme of 8 values and mx as a tree of depth 2 (three independent
    // 3-way extremes, then one), pinned where it is called: without the pin
    // the compiler sinks every extreme of the block to its end, where they
    // form one dependent chain behind the block's last MFMA
    auto ext8t = [&](const f32x16& sb, int half, float mx) __attribute__((always_inline)) {
        const int v = 8 * half;
        auto e3 = [&](float a, float b, float c) __attribute__((always_inline)) {
            return NEG ? fminf(fminf(a, b), c) : fmaxf(fmaxf(a, b), c);
        };
        float r = e3(e3(sb[v], sb[v + 1], sb[v + 2]), e3(sb[v + 3], sb[v + 4], sb[v + 5]), e3(sb[v + 6], sb[v + 7], mx));
        asm volatile("" : "+v"(r));
        return r;
    };
    // after the row extreme of a tile: lazy move of the reference maximum
    auto settle = [&](float mx) __attribute__((always_inline)) {
        const float2 hv = halves(mx);
        mx = NEG ? fminf(hv.x, hv.y) : fmaxf(hv.x, hv.y);
        const float mt = (mx == masked) ? -INFINITY : mx * c2;
        const bool need = mt > m_run + kLazy;
        // lanes that keep their reference scale by 1 (m_run may be -inf
        // there, and -inf - -inf would be NaN); a first finite maximum scales
        // by exp2(-inf) = 0, which only clears zeros
        alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
        m_run = need ? mt : m_run;
        l_run *= alpha;
        rescale = __builtin_amdgcn_ballot_w64(need) != 0;
    };
    auto apply_rescale = [&]() __attribute__((always_inline)) {
        if (rescale) {
            asm volatile("");
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        }
    };

    // One pipeline step: P(t) from scur, O += P(t)·V(t) from vb and, if NEXT,
    // S(t+1) from kb into snew; returns the extreme of the unmasked S(t+1).
    // K operands of the first chunk (S-steps 0 and 1 of block 1), read by the
    // caller ahead of the step's DMA issue so their LDS latency overlaps it
    auto kfirst = [&](const unsigned char* kb, bf16x8 (&kr)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SPC; ++i) kr[i] = kread(kb, i, 1);
    };
    auto main_block = [&](auto next_c, const unsigned char* kb, const unsigned char* vb,
                          f32x16 (&scur)[KB], f32x16 (&snew)[KB], bf16x8 (&kr)[4], auto&& dma) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next_c)::value;
        apply_rescale();
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        float la = l_run, lb = 0.f;
        bf16x8 pb[KS];
        bf16x8 vr[2][2];
        float mx = masked;
        // Ten chunks. Chunk c < 8: the two MFMAs of S(t+1) for block 1 - c/4,
        // S-steps 2(c%4) and 2(c%4)+1 (K read one chunk ahead), and one eighth
        // of P(t). From chunk 2 on, two P(t)·V(t) MFMAs per chunk (P·V step
        // (c-2)/2, d blocks 2((c-2)%2) and 2((c-2)%2)+1, V read one chunk
        // ahead). The extreme of S(t+1) block 1 runs in chunks 6-7, block 0
        // (whose last MFMA issues in chunk 7) in chunk 9.
        auto kst = [](int c, int i) __attribute__((always_inline)) { return SPC * (c & 3) + i; };
        auto kblk = [](int c) __attribute__((always_inline)) { return 1 - (c >> 2); };
        auto vread2 = [&](int c, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
            const int ks = (c - 2) >> 1, db0 = DPC * ((c - 2) & 1);
#pragma unroll
            for (int i = 0; i < DPC; ++i) dst[i] = vop(vb, ks, db0 + i);
        };
#pragma unroll
        for (int c = 0; c < 10; ++c) {
            __builtin_amdgcn_sched_barrier(0);
            if (c == 2) {
                dma();
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (NEXT) {
                if (c + 1 < 8) {
#pragma unroll
                    for (int i = 0; i < SPC; ++i) kr[SPC * ((c + 1) & 1) + i] = kread(kb, kst(c + 1, i), kblk(c + 1));
                }
                if (c < 8) {
                    const int kbs = kblk(c);
#pragma unroll
                    for (int i = 0; i < SPC; ++i) {
                        const f32x16 zero = {};
                        snew[kbs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[SPC * (c & 1) + i], qreg[kst(c, i)],
                                                                            ((c & 3) == 0 && i == 0) ? zero : snew[kbs],
                                                                            0, 0, 0);
                    }
                }
            }
            if (c + 1 >= 2 && c + 1 < 10) vread2(c + 1, vr[(c + 1) & 1]);
            if (c >= 2) {
                const int ks = (c - 2) >> 1, db0 = DPC * ((c - 2) & 1);
#pragma unroll
                for (int i = 0; i < DPC; ++i)
                    oacc[db0 + i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[c & 1][i], pb[ks], oacc[db0 + i], 0, 0, 0);
            }
            if (c < 8) {
                // P(t): k-step ks = c / 2, pairs j = 4*(c%2) and 4*(c%2)+2
                const int ks = c >> 1, kbk = ks >> 1;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int j = 4 * (c & 1) + 2 * jj;
                    const int v0 = 8 * (ks & 1) + j;
                    f32x2 pr = {__builtin_amdgcn_exp2f(fmaf(scur[kbk][v0], c2, -msub)),
                                __builtin_amdgcn_exp2f(fmaf(scur[kbk][v0 + 1], c2, -msub))};
                    const bf16x2 pbf = __builtin_convertvector(pr, bf16x2);
                    if (jj) lb = __builtin_amdgcn_fdot2_f32_bf16(pbf, __builtin_bit_cast(bf16x2, ones), lb, false);
                    else la = __builtin_amdgcn_fdot2_f32_bf16(pbf, __builtin_bit_cast(bf16x2, ones), la, false);
                    pb[ks][j] = pbf[0];
                    pb[ks][j + 1] = pbf[1];
                }
            }
            if constexpr (NEXT) {
                if (c == 6 || c == 7) mx = ext8t(snew[1], c - 6, mx);
                if (c == 9) mx = ext8t(snew[0], 1, ext8t(snew[0], 0, mx));
            }
        }
        l_run = la + lb;
        __builtin_amdgcn_sched_barrier(0);
        return mx;
    };
    // mask of a boundary tile, then its extreme
    auto edge_extreme = [&](f32x16 (&sb)[KB], int j0) __attribute__((always_inline)) {
        asm volatile("");
        float mx = masked;
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk) {
            mask8(sb[kbk], j0, kbk, 0);
            mask8(sb[kbk], j0, kbk, 1);
            mx = ext8(sb[kbk], 1, ext8(sb[kbk], 0, mx));
        }
        return mx;
    };

    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    int pid = 0;   // paged: prefetched page ids of this step's DMA
    auto step = [&](int t, const unsigned char* kb, const unsigned char* vb, unsigned char* kdst,
                    unsigned char* vdst, f32x16 (&scur)[KB], f32x16 (&snew)[KB]) __attribute__((always_inline)) {
        bf16x8 kr[4];
        kfirst(kb, kr);
        auto dma = [&]() __attribute__((always_inline)) {
            if (t + 2 < t_end) issue(krs, t + 2, kdst, false, pid, PAGED);
            issue(vrs, t + 1, vdst, true, pid, PAGED);
            if constexpr (PAGED) pid = page_ids(t + 3, t + 2);
        };
        float mx = main_block(T{}, kb, vb, scur, snew, kr, dma);
        if (is_edge(t + 1)) mx = edge_extreme(snew, (t + 1) * BN);
        settle(mx);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    // the wave's last tile u (V(u) in vb): P(u)·V(u) only
    auto last_step = [&](int u, const unsigned char* vb, unsigned char* kdst, unsigned char* vdst,
                         f32x16 (&scur)[KB]) __attribute__((always_inline)) {
        if (u + 2 < t_end) issue(krs, u + 2, kdst, false, pid, PAGED);
        if (u + 1 < t_end) issue(vrs, u + 1, vdst, true, pid, PAGED);
        bf16x8 kr[4];
        main_block(F{}, k_lds0, vb, scur, scur, kr, []() {});
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    // a step after the wave's last tile: its share of the DMA and the barrier
    auto idle_step = [&](int u) __attribute__((always_inline)) {
        const bool odd = (u - t_begin) & 1;
        if (u + 2 < t_end) issue(krs, u + 2, odd ? k_lds1 : k_lds0, false);
        if (u + 1 < t_end) issue(vrs, u + 1, odd ? v_lds0 : v_lds1, true);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // A wave stops computing after its last visible tile (it still issues its
    // share of the DMA and meets every barrier). Waves whose rows start after
    // the group's first tiles compute those fully masked tiles, which add
    // exact zeros.
    f32x16 sA[KB], sB[KB];
    // Q rows into registers, then the first tiles K(t0), K(t0+1) and V(t0)
    // (their buffers are all free), so the item waits for memory once
    {
        const bool ok = qrow < Sq;
        const uint16_t* qp = Q + qo_base + (size_t)(ok ? qrow : 0) * D + 8 * hh;
#pragma unroll
        for (int st = 0; st < DS; ++st) {
            uint4 x = ok ? ld_global16(qp + 16 * st) : make_uint4(0, 0, 0, 0);
            qreg[st] = as_bf16x8(x);
        }
    }
    issue(krs, t_begin, k_lds0, false);
    if (t_begin + 1 < t_end) issue(krs, t_begin + 1, k_lds1, false);
    issue(vrs, t_begin, v_lds0, true);
    if constexpr (PAGED) pid = page_ids(t_begin + 2, t_begin + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
#pragma unroll
        for (int st = 0; st < DS; ++st)
#pragma unroll
            for (int kbk = 0; kbk < KB; ++kbk) {
                const f32x16 zero = {};
                sA[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(k_lds0, st, kbk), qreg[st],
                                                                  st == 0 ? zero : sA[kbk], 0, 0, 0);
            }
        float mx = masked;
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk) mx = ext8(sA[kbk], 1, ext8(sA[kbk], 0, mx));
        if (is_edge(t_begin)) mx = edge_extreme(sA, t_begin * BN);
        settle(mx);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // tile t: K(t+1) in k_lds[(t - t_begin + 1) & 1], V(t) in v_lds[(t - t_begin) & 1]
    int t = t_begin;
    if (wt_hi >= t_begin) {
        for (; t + 1 < wt_hi; t += 2) {
            step(t, k_lds1, v_lds0, k_lds0, v_lds1, sA, sB);
            step(t + 1, k_lds0, v_lds1, k_lds1, v_lds0, sB, sA);
        }
        if (t < wt_hi) {
            step(t, k_lds1, v_lds0, k_lds0, v_lds1, sA, sB);
            last_step(t + 1, v_lds1, k_lds1, v_lds0, sB);
            t += 2;
        } else {
            last_step(t, v_lds0, k_lds0, v_lds1, sA);
            t += 1;
        }
    }
    for (; t < t_end; ++t) idle_step(t);

    if (wr0 >= Sq) return;
    const float2 lh = halves(l_run);
    const float inv = 1.f / (lh.x + lh.y);
    // log-sum-exp of the scaled logits, natural log: sum_j exp(scale s_j)
    // = 2^m_ref * l with m_ref the reference maximum in log2 units
    if (LSE != nullptr && hh == 0 && qrow < Sq)
        LSE[((size_t)b * Hq + h) * Sq + qrow] = (m_run + __log2f(lh.x + lh.y)) * 0.69314718055994531f;
    // The wave's 32 x D output block goes out through LDS (the K/V buffers
    // are free after the last barrier; 8 KiB per wave): from the accumulator
    // layout (per 16-byte column chunk, 16 bytes of each of 32 rows) to
    // whole rows, so every store instruction writes four contiguous rows.
    // Chunks are XOR-swizzled by (row & 15) so both sides spread over banks.
    unsigned char* stage = (wave >> 1) == 0 ? k_lds0 : (wave >> 1) == 1 ? k_lds1 : (wave >> 1) == 2 ? v_lds0 : v_lds1;
    stage += (wave & 1) * (32 * D * 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x2 a = {oacc[db][4 * r + 0] * inv, oacc[db][4 * r + 1] * inv};
            f32x2 c = {oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv};
            uint2 st;
            st.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2));
            st.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(c, bf16x2));
            const int chunk = (4 * db + r) ^ (ln & (CPR - 1));
            *reinterpret_cast<uint2*>(stage + ln * (D * 2) + chunk * 16 + hh * 8) = st;
        }
    wave_lds_fence();
    const int cl = lane % CPR;
#pragma unroll
    for (int i = 0; i < CPR / 2; ++i) {
        const int row = i * (64 / CPR) + lane / CPR;
        const uint4 x = *reinterpret_cast<const uint4*>(stage + row * (D * 2) + ((cl ^ (row & (CPR - 1))) << 4));
        if (wr0 + row < Sq) *reinterpret_cast<uint4*>(O + qo_base + (size_t)(wr0 + row) * D + 8 * cl) = x;
    }
}

template <int NW, int D, bool NEG, bool PAGED>
hipError_t launch_pipe(const PrefillArgs& a, hipStream_t stream) {
    const int nqt = (a.Sq + 32 * NW - 1) / (32 * NW);
    const long long nitems = (long long)a.B * a.Hq * nqt;
    const Deal deal = make_deal(nitems, (long long)(a.Hq / a.Hkv) * nqt, a.Hq / a.Hkv, PAGED);
    if (!grid_fits(deal.grid, 64 * NW)) return hipErrorInvalidValue;
    float c2 = a.scale * 1.4426950408889634f;
    if (c2 == 0.f) c2 = 1e-30f;
    int ps_log2 = 0;
    while ((1 << ps_log2) < a.page_size) ++ps_log2;
    // causal items, one run of whole groups per XCD: order by weight (four
    // waves: two workgroups per CU, eight waves: one)
    const int pair = PAGED ? 0
                           : balance_arg(nitems, deal.chunk, (long long)(a.Hq / a.Hkv) * nqt, deal.grid, a.causal,
                                         a.num_cu, NW == 8 ? 1 : D == 64 ? 3 : 2);
    if (log_enabled())
        log_dispatch("prefill_pipe_kernel<%d,%d,%s,%s> B=%d Hq=%d Hkv=%d Sq=%d Sk=%d causal=%d window=%d%s: "
                     "grid %lld x %d threads, %lld items of %d rows, chunk %lld, balance %d",
                     NW, D, NEG ? "neg" : "pos", PAGED ? "paged" : "contiguous", a.B, a.Hq, a.Hkv, a.Sq, a.Sk,
                     a.causal, a.window, a.lse ? " +lse" : "", deal.grid, 64 * NW, nitems, 32 * NW, deal.chunk,
                     pair);
    hipLaunchKernelGGL((prefill_pipe_kernel<NW, D, NEG, PAGED>), dim3((unsigned)deal.grid), dim3(64 * NW), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                       a.Hq, a.Hkv, a.Sq, a.Sk, c2, a.causal, a.window, nqt, (int)nitems, (int)deal.chunk, pair,
                       a.page_table, a.seq_lens, ps_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const bool neg = a.scale < 0.f;
    // D = 128: 256-row workgroups (eight waves) unless that leaves fewer than
    // two workgroups per CU, or the keys are at most 2048, then 128-row ones
    // (four waves, two per CU): a short item spends much of its time in the
    // diagonal tiles (half as many with 128 rows) and in its start, which the
    // second workgroup of the CU overlaps (16 x 32 heads x 1024 tokens causal:
    // 524 -> 637 TFLOP/s; at 4096 keys the eight-wave kernel is ahead)
    const long long wg256 = (long long)a.B * a.Hq * ((a.Sq + 255) / 256);
    const bool small = wg256 < 2LL * 256 || (a.page_table == nullptr && a.Sk <= 2048);
    if (a.page_table != nullptr) {  // paged K/V
        if (a.D == 64) return neg ? launch_pipe<4, 64, true, true>(a, stream) : launch_pipe<4, 64, false, true>(a, stream);
        if (small) return neg ? launch_pipe<4, 128, true, true>(a, stream) : launch_pipe<4, 128, false, true>(a, stream);
        return neg ? launch_pipe<8, 128, true, true>(a, stream) : launch_pipe<8, 128, false, true>(a, stream);
    }
    if (a.D == 128) {
        if (small) return neg ? launch_pipe<4, 128, true, false>(a, stream) : launch_pipe<4, 128, false, false>(a, stream);
        return neg ? launch_pipe<8, 128, true, false>(a, stream) : launch_pipe<8, 128, false, false>(a, stream);
    }
    return neg ? launch_pipe<4, 64, true, false>(a, stream) : launch_pipe<4, 64, false, false>(a, stream);
}

}  // namespace attn
