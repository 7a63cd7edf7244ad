/*
 * attn.h — C ABI of libattn.so: fused scaled-dot-product attention on MI355X
 * (gfx950), prefill and paged single-token decode.
 *
 * The operation (web pages, cited by title and section):
 *   O = softmax(Q K^T * scale) V, row by row, with masked logits set to -inf
 *   before the softmax and the row maximum subtracted before exponentiating
 *   ("Attention 机制详解：从 Self-Attention 到 Multi-Query Attention" §2.1–2.2;
 *   "拆开 LLM（二）：手撕注意力", sections "手撕三种打分函数" and
 *   "从对齐机器到 self-attention"). It is computed tile by tile with an online
 *   softmax so the Sq x Sk score matrix never reaches memory ("Attention 机制
 *   详解" §7; "拆开 LLM（二）", section on FlashAttention: the result is exact,
 *   not an approximation).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *     row-major in the layout stated per call, 16-byte aligned. The library
 *     never frees or retains them.
 *   - Calls are asynchronous: they validate the arguments on the host (before
 *     any HIP call, so every error below is reported without touching a GPU),
 *     enqueue kernels on `stream` and return. Faults inside a kernel surface
 *     at the caller's next synchronisation of that stream.
 *   - Return value: ATTN_OK (0) or a negative ATTN_ERR_* code; nothing is
 *     enqueued when an error is returned. No C++ exception crosses the ABI.
 *   - GQA/MQA: Hq must be a multiple of Hkv; query head h reads K/V head
 *     h / (Hq / Hkv) ("Attention 机制详解" §5.2, repeat_interleave order).
 *     Hkv == Hq is plain multi-head attention, Hkv == 1 is multi-query.
 *   - A zero batch (B == 0), or Sq == 0 for prefill, is a valid empty call.
 *   - Graph capture: a call enqueues kernels only (no memset, copy or host
 *     synchronisation). The one allocation is the workspace of the decode and
 *     backward calls, kept per (device, stream) and grown on demand. A buffer
 *     that a larger request replaces is retired, not freed, so kernels still
 *     in flight and graphs that captured an earlier call keep a valid buffer
 *     until attn_release. The workspace never grows while `stream` is being
 *     captured (ATTN_ERR_CAPTURE): run the calls once on the capture stream
 *     with the largest shapes to be captured first. A graph that captured a
 *     decode or backward call must not be replayed after attn_release.
 *   - Threads: every entry point may be called from several host threads.
 *     The workspace lock is held from its size check until the call's
 *     kernels are enqueued; two calls that share a (device, stream) run in
 *     the order they were enqueued.
 *   - Logging: the library prints nothing, except with ATTN_LOG set to a
 *     value other than "" or "0" in the environment (read once per process):
 *     then each kernel launch decision (kernel and template arguments,
 *     shape, grid, work split) is one "[attn] ..." line on stderr.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,     /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,    /* a size is negative or zero where it must be >= 1,
                               causal with Sq > Sk, Sq > 2^30, an element count
                               overflows 64-bit addressing, one (batch, kv
                               head) slice of K/V exceeds 2^31 bytes in float32
                               (Sk * D * 4 >= 2^31), or the launch grid would
                               exceed the dispatch limit: prefill B * Hq *
                               ceil(Sq / 128) > 2^22 (bf16) or B * Hq *
                               ceil(Sq / 16) > 2^23 (float32) */
    ATTN_ERR_HEADS = -3,    /* Hq < 1, Hkv < 1 or Hq % Hkv != 0 */
    ATTN_ERR_HEADDIM = -4,  /* D is not 64 or 128 */
    ATTN_ERR_MASK = -5,     /* causal not 0/1, window < 0, or (prefill) window > 0
                               without causal */
    ATTN_ERR_SCALE = -6,    /* scale is NaN or infinite */
    ATTN_ERR_PAGE = -7,     /* page_size is not a power of two in [8, 256] */
    ATTN_ERR_ALIGN = -8,    /* a tensor pointer is not 16-byte aligned */
    ATTN_ERR_NOMEM = -9,    /* the decode workspace could not be allocated */
    ATTN_ERR_HIP = -10,     /* a HIP runtime call or kernel launch failed */
    ATTN_ERR_FULL = -11,    /* the page pool has too few free pages */
    ATTN_ERR_SEQ = -12,     /* a sequence id the page pool does not hold */
    ATTN_ERR_CAPTURE = -13, /* the decode/backward workspace would have to grow
                               while `stream` is being captured into a graph */
    ATTN_ERR_SCRATCH = -14  /* attn_decode_paged_noalloc: the call needs more
                               than its fixed scratch (B * Hq * (D + 2) * 4 bytes
                               > 16 MiB) */
};

/*
 * attn_fwd — prefill attention, bfloat16 in and out, float32 accumulation.
 *
 *   q, o : [B, Hq, Sq, D] bfloat16      k, v : [B, Hkv, Sk, D] bfloat16
 *   scale: multiplies Q K^T (typically 1/sqrt(D), "Attention 机制详解" §2.1);
 *          any finite value, 0 gives the mean of the visible V rows.
 *   causal: 1 = each query sees only keys at or before its position
 *          ("拆开 LLM（二）", causal mask = lower triangle). When Sq < Sk the
 *          queries are the LAST Sq positions: row i sits at position
 *          i + Sk - Sq (bottom-right alignment, which makes a one-token call
 *          equal to one decode step over a cache of Sk tokens).
 *   window: 0 = no window; W > 0 (requires causal) = each query sees only the
 *          W most recent keys, its own position included ("LLM 核心技术：
 *          Attention 机制的实现与优化", sliding-window section; "拆开 LLM（二）",
 *          exercise keeping the last 256 cache entries).
 *   The probabilities P are rounded to bfloat16 before P·V; O is rounded to
 *   bfloat16 (round-to-nearest-even) once, after the final normalisation.
 *   o must not overlap q, k or v.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o,
             int B, int Hq, int Hkv, int Sq, int Sk, int D,
             float scale, int causal, int window, hipStream_t stream);

/*
 * attn_fwd_f32 — the same operation and arguments with float32 tensors and
 * float32 arithmetic throughout (no reduced-precision rounding of Q, K, P or
 * V). Intended for accuracy checks against a float64 reference.
 */
int attn_fwd_f32(const void* q, const void* k, const void* v, void* o,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D,
                 float scale, int causal, int window, hipStream_t stream);

/*
 * attn_fwd_lse, attn_fwd_f32_lse — attn_fwd / attn_fwd_f32 that also return
 * the log-sum-exp of each query row, the second output of the FlashAttention
 * forward in "Attention From Scratch" (FlashAttention module: output and lse),
 * used to merge attention computed over separate key ranges.
 *   lse : [B, Hq, Sq] float32, device, 4-byte aligned, caller-owned:
 *         lse[b,h,i] = ln( sum over the keys j visible to row i of
 *         exp(scale * q_i . k_j) ), natural logarithm. In the bf16 call the
 *         sum adds the bf16-rounded probabilities that also weight V (relative
 *         error below 2^-8 of the sum, so |error| of lse < 2^-8); the f32 call
 *         keeps float32 throughout. o is identical to the plain call's.
 *   Errors: those of attn_fwd, and NULL / ALIGN for lse. Empty calls (B == 0
 *   or Sq == 0) write nothing and accept a NULL lse.
 */
int attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D,
                 float scale, int causal, int window, hipStream_t stream);
int attn_fwd_f32_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     float scale, int causal, int window, hipStream_t stream);

/*
 * attn_fwd_paged — prefill of Sq new tokens per sequence against a paged KV
 * cache (chunked prefill): the prefill of attn_fwd with K and V read through
 * the page table of attn_decode_paged instead of from contiguous tensors
 * ("LLM 核心技术", PagedAttention section: attention reads the cache through
 * the page table; "拆开 LLM（二）", KV-cache section: new tokens attend to the
 * cached ones).
 *   q, o        : [B, Hq, Sq, D] bfloat16, the Sq newest tokens of each
 *                 sequence, whose k and v are already in the cache.
 *   k_pool, v_pool, page_table, seq_lens, page_size : as in
 *                 attn_decode_paged; sequence b has Sk_b = seq_lens[b] cached
 *                 tokens and query row i sits at position Sk_b - Sq + i
 *                 (bottom-right alignment, as in attn_fwd with Sq <= Sk).
 *   lse         : NULL, or [B, Hq, Sq] float32 receiving the log-sum-exp of
 *                 each row as in attn_fwd_lse.
 *   D is 64 or 128 (ATTN_ERR_HEADDIM otherwise). causal / window as in
 *   attn_fwd. Device-side preconditions: those of attn_decode_paged, and
 *   seq_lens[b] >= Sq when causal. Slots at or past seq_lens[b] are never
 *   used (they may hold NaN). Errors: those of attn_fwd and attn_decode_paged
 *   for the same arguments; B == 0 or Sq == 0 is a no-op.
 */
int attn_fwd_paged(const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* page_table, const int32_t* seq_lens, void* o, float* lse,
                   int B, int Hq, int Hkv, int Sq, int D, int page_size,
                   float scale, int causal, int window, hipStream_t stream);

/*
 * attn_decode_paged — one decode step: each of B sequences has one new query
 * token that attends, without a mask, to every token of its paged KV cache
 * ("拆开 LLM（二）", KV-cache section: the new token's k and v are appended
 * first, then it attends over all cached positions; "LLM 核心技术",
 * PagedAttention section: the cache is stored in fixed-size pages of a global
 * pool and reached through a page table).
 *
 *   q, o        : [B, Hq, D] bfloat16, one token per sequence.
 *   k_pool,
 *   v_pool      : [num_pages, Hkv, page_size, D] bfloat16; each (page, head)
 *                 is one contiguous page_size x D tile.
 *   seq_lens    : [B] int32, device memory: tokens cached for sequence b,
 *                 the current token included; every entry must be >= 1.
 *   page_table  : int32, device memory, ragged: sequence b owns the
 *                 ceil(seq_lens[b] / page_size) consecutive entries starting
 *                 at off_b = sum over j < b of ceil(seq_lens[j] / page_size);
 *                 entry off_b + p is the physical page of logical page p.
 *                 Token t of sequence b is slot t % page_size of logical page
 *                 t / page_size. Slots at or past seq_lens[b] are never read
 *                 (they may hold anything, NaN included).
 *   page_size   : power of two in [8, 256].
 *   Device-side preconditions the host cannot check without synchronising:
 *   seq_lens[b] >= 1 and every used page id in [0, num_pages); violating
 *   them is undefined behaviour.
 *   The split-context partial results live in a library-owned workspace,
 *   allocated on first use per (device, stream) and grown as needed; calls on
 *   different streams never share a workspace. P is rounded to bfloat16
 *   before P·V, as in attn_fwd.
 *   Errors: NULL; SHAPE (B < 0, B > 65535, Hq > 65535 or B * Hq > 2^24: the
 *   launch grids index sequences and head groups in 16-bit grid dimensions
 *   and the merge runs one workgroup per (sequence, query head)); HEADS;
 *   HEADDIM; PAGE; SCALE; ALIGN (16 bytes for tensors, 4 for the int32
 *   arrays); NOMEM and CAPTURE for the workspace; HIP. B == 0 is a no-op.
 */
int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* page_table, const int32_t* seq_lens,
                      int B, int Hq, int Hkv, int D, int page_size,
                      float scale, void* o, hipStream_t stream);

/*
 * attn_decode_paged_noalloc — attn_decode_paged that allocates nothing, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * layouts, preconditions and result as attn_decode_paged (the same kernels).
 *   The split-context partials go to a fixed scratch array of 16 MiB in
 *   device memory instead of the library's workspace; each GPU the library
 *   runs on holds its own copy from the first call on that device until the
 *   process ends. The call makes no hipMalloc or hipFree and no other
 *   allocating call; the array's address is looked up once per device on the
 *   first call there, with that device current.
 *   Limit: B * Hq * (D + 2) * 4 bytes must fit the 16 MiB (one context split
 *   per (sequence, query head); B * Hq <= 32263 at D = 128), else
 *   ATTN_ERR_SCRATCH with nothing enqueued. Beyond one split the call takes
 *   as many splits as attn_decode_paged would, up to what the scratch holds.
 *   Every call on one GPU shares that GPU's array and leaves its partials in
 *   it: calls that overlap on one GPU (several streams, or several host
 *   threads) race and give undefined results; serialise them.
 *   Errors: those of attn_decode_paged (CAPTURE and NOMEM cannot occur), and
 *   SCRATCH.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* page_table, const int32_t* seq_lens,
                              int B, int Hq, int Hkv, int D, int page_size,
                              float scale, void* o, hipStream_t stream);

/*
 * attn_decode_paged_window — the same decode step restricted to a sliding
 * window: each sequence's query attends only to its `window` most recent
 * cached tokens, positions max(0, seq_lens[b] - window) .. seq_lens[b] - 1,
 * the current token included ("拆开 LLM（二）：手撕注意力", exercise that keeps
 * only the last 256 cache entries; "LLM 核心技术：Attention 机制的实现与优化",
 * sliding-window section: each token attends to the W previous ones).
 *   window: >= 0; 0 means no window (identical to attn_decode_paged), a window
 *   at least seq_lens[b] sees the whole sequence. window < 0 is
 *   ATTN_ERR_MASK. Every other argument, layout, precondition and the
 *   workspace are those of attn_decode_paged; pages wholly before the window
 *   are never read.
 */
int attn_decode_paged_window(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* page_table, const int32_t* seq_lens,
                             int B, int Hq, int Hkv, int D, int page_size,
                             float scale, int window, void* o, hipStream_t stream);

/*
 * attn_kv_append — write the new token's k and v into the paged cache, the
 * step that precedes attention in a decode ("拆开 LLM（二）：手撕注意力",
 * KV-cache section: the new key and value are appended, then the token
 * attends to every cached position; "LLM 核心技术", PagedAttention section).
 *
 *   k_new, v_new : [B, Hkv, D] bfloat16, one token per sequence.
 *   k_pool, v_pool, page_table, seq_lens, page_size : as in
 *                  attn_decode_paged. seq_lens[b] already counts the new
 *                  token: it is written to position seq_lens[b] - 1, slot
 *                  (seq_lens[b] - 1) % page_size of physical page
 *                  page_table[off_b + (seq_lens[b] - 1) / page_size]. Nothing
 *                  else in the pools changes.
 *   The page holding that position must already be in the table (see
 *   attn_pages_resize); the device-side preconditions of attn_decode_paged
 *   apply. Sequences must not share physical pages.
 *   Errors: NULL, SHAPE (B < 0 or B > 2^24), HEADS (Hkv < 1), HEADDIM, PAGE, ALIGN
 *   (16 bytes for tensors, 4 for the int32 arrays), HIP. B == 0 is a no-op.
 */
int attn_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                   const int32_t* page_table, const int32_t* seq_lens,
                   int B, int Hkv, int D, int page_size, hipStream_t stream);

/*
 * Page pool — host-side allocator of the physical pages of a paged KV cache
 * ("LLM 核心技术", PagedAttention section; "Attention From Scratch", paged
 * KV cache: fixed-size pages from one global pool, handed to sequences on
 * demand and returned when they shrink or end). Pure host code: no HIP call,
 * no device memory. Each call locks the pool, so one pool may be shared by
 * threads. The pool owns no cache memory; it only hands out page ids
 * 0 .. num_pages - 1 of pools the caller allocates.
 *
 * attn_pages_create  — a pool of num_pages (>= 1, else SHAPE) free pages of
 *                      page_size tokens (power of two in [8, 256], else PAGE);
 *                      *out receives the handle (NULL out: NULL; NOMEM).
 * attn_pages_destroy — frees the handle (NULL is a no-op).
 * attn_pages_resize  — sets sequence seq_id (any int64 key; created on first
 *                      use) to len >= 0 tokens (SHAPE if negative): it then
 *                      owns ceil(len / page_size) pages. Missing pages are
 *                      taken from the free list and appended in logical
 *                      order; surplus pages leave from the end and return to
 *                      the free list; len == 0 releases every page and drops
 *                      the sequence. FULL (state unchanged) if too few pages
 *                      are free.
 * attn_pages_free_count — free pages, or NULL for a NULL pool.
 * attn_pages_table   — for the n sequences seq_ids[0..n-1], in that order,
 *                      writes seq_lens[i] and the ragged page table of
 *                      attn_decode_paged (each sequence's pages in logical
 *                      order, sequences back to back); *table_len receives the
 *                      number of entries. SEQ for an unknown id; SHAPE (with
 *                      *table_len set) if table_cap is smaller than needed.
 *                      Host pointers; copy the arrays to the device for the
 *                      kernels.
 */
typedef struct attn_page_pool attn_page_pool;
int attn_pages_create(int num_pages, int page_size, attn_page_pool** out);
void attn_pages_destroy(attn_page_pool* pool);
int attn_pages_resize(attn_page_pool* pool, int64_t seq_id, int len);
int attn_pages_free_count(const attn_page_pool* pool);
int attn_pages_table(const attn_page_pool* pool, const int64_t* seq_ids, int n, int32_t* page_table,
                     int64_t table_cap, int32_t* seq_lens, int64_t* table_len);

/*
 * attn_bwd — backward pass of attn_fwd: the gradients dq, dk, dv of
 * L = sum(dout * o) for o = attn_fwd(q, k, v, ...). The pages name the
 * backward only through FlashAttention's recomputation ("Attention From
 * Scratch", 进阶篇 §5; "LLM 核心技术", section 底层算子优化：FlashAttention):
 * the weights P are recomputed from q, k and the forward's lse instead of
 * being stored. With S = scale * q k^T (masked as in attn_fwd) and
 * P = exp(S - lse): dv = P^T dout, dS = P * (dout v^T - rowsum(dout * o)),
 * dq = scale * dS k, dk = scale * dS^T q; dk and dv of a K/V head sum over
 * the query heads that read it (GQA).
 *   q, o, dout, dq : [B, Hq, Sq, D] bfloat16, device, 16-byte aligned.
 *   k, v, dk, dv   : [B, Hkv, Sk, D] bfloat16, device, 16-byte aligned.
 *   lse            : [B, Hq, Sq] float32, device, 4-byte aligned: the lse that
 *                    attn_fwd_lse returned with this o (natural logarithm).
 *   dq, dk, dv are written in full (keys no query sees get zero gradients);
 *   they must not overlap the inputs. Arithmetic: bf16 MFMA products with
 *   float32 accumulation; P and dS are rounded to bf16 as MFMA operands, and
 *   rowsum(dout * o) uses the bf16 o.
 *   Scratch, in the per-(device, stream) workspace that attn_decode_paged
 *   also uses (grown on demand, freed by attn_release): 2 * B * Hq * Sq
 *   floats (rowsum(dout * o) and the lse in log2 units), transposed copies of
 *   q and dout (2 * B * Hq * Sq * D bf16, Sq rounded up to 32), and, when the
 *   (batch, kv head, 256-key) blocks are too few to fill the device, float32
 *   partial dk and dv of up to 16 runs per block (2 * runs * B * Hkv * Sk * D
 *   floats), summed in a fixed order: the result is bit-reproducible.
 *   Errors: those of attn_fwd for the same sizes, plus NULL / ALIGN for the
 *   extra pointers, NOMEM and CAPTURE for the workspace, and SHAPE when
 *   Sq * D or Sk * D exceeds 2^29 (one head's rows are addressed with 32-bit
 *   offsets) or B * Hq * ceil(Sq / 128) or B * Hkv * ceil(Sk / 256) exceeds
 *   2^22 (launch grids).
 *   B == 0 is a no-op; Sq == 0 writes zero dk and dv and then accepts NULL
 *   for q, k, v, o, dout, lse and dq.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int D,
             float scale, int causal, int window, hipStream_t stream);

/* attn_strerror — static, never-NULL description of a status code. */
const char* attn_strerror(int status);

/*
 * attn_release — synchronise every device the library used and free the
 * decode workspaces. Idempotent; later calls allocate again on demand.
 */
void attn_release(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
