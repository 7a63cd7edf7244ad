"""Plain float64 attention, written straight from the definition (test infrastructure).

Sources (web pages; cited by title and section):

* "Attention 机制详解：从 Self-Attention 到 Multi-Query Attention" (guijiagi.com),
  §2.1 (the formula softmax(QK^T / sqrt(d_k)) V), §2.2 (masked positions get
  -inf before the softmax), §5.2 (GQA: each K/V head serves n_heads/n_kv_heads
  consecutive query heads, via repeat_interleave on the head axis).
* "拆开 LLM（二）：手撕注意力" (blog.kerro.cn), section "手撕三种打分函数"
  (softmax with the row maximum subtracted first), section
  "从对齐机器到 self-attention" (logits -> mask with -inf -> softmax -> weights
  times V; the causal mask is lower-triangular, True = visible), section
  "KV cache" (a new token appends its k, v, then attends over every cached
  position with no mask), section "试一试" (a window that keeps the last W
  positions, the current one included).
* "LLM 核心技术：Attention 机制的实现与优化" (zeeklog.com), sections on SWA
  (each token sees only the previous W tokens) and PagedAttention (the KV cache
  lives in fixed-size pages of a global pool, reached through a per-sequence
  page table).

Nothing here is blocked, fused or reordered beyond the definition: for each
(batch, query head) the full score matrix is formed with one matrix product,
masked, normalised row by row and multiplied by V. Rows are independent, so a
row subset (``attention_rows``) or row chunks give the same numbers as the full
matrix.

Readings taken where the pages leave a point open:

* Window: key j is visible to query position p iff p - W < j <= p (W keys,
  the query's own position included); ``window == 0`` means no window. Only
  causal windows appear on the pages, so a window requires ``causal``.
* Causal alignment when Sq != Sk: bottom-right. Query row i sits at absolute
  position i + (Sk - Sq); this is the only alignment under which decoding one
  token against the cache equals the last row of a full causal pass.
* GQA: query head h reads K/V head h // (Hq // Hkv).
* Paged cache: ``pool[page, kv_head, slot, d]``; the page table is the ragged
  concatenation of every sequence's pages in logical order, sequence b owning
  ceil(seq_lens[b] / page_size) entries; tokens at or beyond seq_lens[b] are
  never read.

This module is test infrastructure. It is imported by the tests, by the smoke
check and by the CPU-baseline leg of the benchmark, never by the library.
"""

import numpy as np


def visible(Sq, Sk, causal, window):
    """Boolean [Sq, Sk] visibility of key j to query row i.

    Causal masking keeps keys at or before the query's position (lower
    triangle, "拆开 LLM（二）", section "从对齐机器到 self-attention"); a window
    W additionally drops keys more than W - 1 positions back ("LLM 核心技术",
    section SWA). Query row i is at position i + Sk - Sq (bottom-right).
    """
    pos = np.arange(Sq)[:, None] + (Sk - Sq)
    j = np.arange(Sk)[None, :]
    vis = np.ones((Sq, Sk), dtype=bool)
    if causal:
        vis &= j <= pos
    if window > 0:
        if not causal:
            raise ValueError("a window is only defined together with causal masking")
        vis &= j > pos - window
    return vis


def softmax_rows(x):
    """Row softmax with the row maximum subtracted first.

    "拆开 LLM（二）", section "手撕三种打分函数": shifting a row by a constant
    does not change its softmax, and after subtracting the maximum the largest
    exponent is exp(0) = 1, so nothing overflows; -inf entries become exactly 0.
    """
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def _scores(qrows, k, scale, vis_rows):
    # "Attention 机制详解" §2.2: scores = Q K^T scaled, masked entries -> -inf
    # before the softmax ("拆开 LLM（二）" pitfalls 1 and 2: -inf, never 0, and
    # never after the softmax).
    s = (qrows @ k.T) * scale
    return np.where(vis_rows, s, -np.inf)


def _kv_head(h, Hq, Hkv):
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    # "Attention 机制详解" §5.2: repeat_interleave(n_rep) on the head axis, so
    # query head h uses K/V head h // n_rep.
    return h // (Hq // Hkv)


def attention_weights(q, k, scale, causal=False, window=0):
    """Softmax weights P for one head: q [Sq, D], k [Sk, D] -> [Sq, Sk]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vis = visible(q.shape[0], k.shape[0], causal, window)
    return softmax_rows(_scores(q, k, scale, vis))


def attention_rows(q, k, v, b, h, rows, scale, causal=False, window=0):
    """Output rows ``rows`` of query head h in batch b, as float64 [len(rows), D].

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D]. Same arithmetic as ``attention``
    restricted to the listed rows (each row of the softmax is independent).
    """
    Sq, Sk = q.shape[2], k.shape[2]
    g = _kv_head(h, q.shape[1], k.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    qr = np.asarray(q[b, h][rows], dtype=np.float64)
    kb = np.asarray(k[b, g], dtype=np.float64)
    vb = np.asarray(v[b, g], dtype=np.float64)
    vis = visible(Sq, Sk, causal, window)[rows]
    p = softmax_rows(_scores(qr, kb, scale, vis))
    return p @ vb


def attention(q, k, v, scale, causal=False, window=0, row_chunk=2048):
    """Full attention output, float64 [B, Hq, Sq, D].

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D] (any real dtype; converted to
    float64 exactly). For every (b, h): O = softmax(mask(Q K^T * scale)) V,
    "Attention 机制详解" §2.1–2.2. ``row_chunk`` only bounds memory.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    out = np.empty((B, Hq, Sq, v.shape[3]), dtype=np.float64)
    vis = visible(Sq, Sk, causal, window)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kb = np.asarray(k[b, g], dtype=np.float64)
            vb = np.asarray(v[b, g], dtype=np.float64)
            for r0 in range(0, Sq, row_chunk):
                r1 = min(Sq, r0 + row_chunk)
                qr = np.asarray(q[b, h, r0:r1], dtype=np.float64)
                p = softmax_rows(_scores(qr, kb, scale, vis[r0:r1]))
                out[b, h, r0:r1] = p @ vb
    return out


def sequence_pages(seq_lens, page_size):
    """(first, count) of each sequence's entries in the ragged page table.

    Sequence b owns ceil(seq_lens[b] / page_size) consecutive entries, after
    those of sequences 0 .. b-1 ("Attention From Scratch", 学习路径 §6: a page
    table records each sequence's pages).
    """
    counts = [(int(n) + page_size - 1) // page_size for n in seq_lens]
    firsts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64) if counts else []
    return list(zip([int(f) for f in firsts], counts))


def gather_sequence(pool, page_table, seq_lens, page_size, b):
    """Contiguous [Hkv, n, D] float64 K (or V) of sequence b, n = seq_lens[b].

    Logical page p of sequence b is physical page page_table[first_b + p];
    token t lives at pool[page, :, t % page_size, :] ("LLM 核心技术", section
    PagedAttention: a page table maps the logical cache onto non-contiguous
    physical blocks). Pages are concatenated in logical order and cut at n.
    """
    first, count = sequence_pages(seq_lens, page_size)[b]
    n = int(seq_lens[b])
    phys = np.asarray(page_table[first:first + count], dtype=np.int64)
    blocks = np.asarray(pool[phys], dtype=np.float64)  # [count, Hkv, ps, D]
    flat = blocks.transpose(1, 0, 2, 3).reshape(blocks.shape[1], count * page_size, -1)
    return flat[:, :n, :]


def decode_paged(q, k_pool, v_pool, page_table, seq_lens, page_size, scale):
    """One decode step over a paged cache, float64 [B, Hq, D].

    q: [B, Hq, D] (the new token of each sequence, whose k, v are already in
    the cache); pools: [num_pages, Hkv, page_size, D]. The new token attends
    to every cached position 0 .. seq_lens[b]-1 with no mask ("拆开 LLM（二）",
    section "KV cache").
    """
    B, Hq, D = q.shape
    out = np.empty((B, Hq, v_pool.shape[3]), dtype=np.float64)
    for b in range(B):
        kb = gather_sequence(k_pool, page_table, seq_lens, page_size, b)[None]
        vb = gather_sequence(v_pool, page_table, seq_lens, page_size, b)[None]
        qb = np.asarray(q[b], dtype=np.float64)[None, :, None, :]
        out[b] = attention(qb, kb, vb, scale, causal=False, window=0)[0, :, 0, :]
    return out


def decode_paged_window(q, k_pool, v_pool, page_table, seq_lens, page_size, scale, window):
    """decode_paged restricted to the `window` most recent cached tokens,
    float64 [B, Hq, D]; window 0 means no window.

    The new token sits at position n-1 of a cache of n tokens and sees
    positions n-window .. n-1 ("拆开 LLM（二）", exercise that keeps only the
    last 256 cache entries; "LLM 核心技术", sliding-window section). This is
    the causal, windowed attention of one query placed at the end of the
    gathered sequence (bottom-right alignment, see `visible`).
    """
    B, Hq, D = q.shape
    out = np.empty((B, Hq, v_pool.shape[3]), dtype=np.float64)
    for b in range(B):
        kb = gather_sequence(k_pool, page_table, seq_lens, page_size, b)[None]
        vb = gather_sequence(v_pool, page_table, seq_lens, page_size, b)[None]
        qb = np.asarray(q[b], dtype=np.float64)[None, :, None, :]
        out[b] = attention(qb, kb, vb, scale, causal=True, window=int(window))[0, :, 0, :]
    return out


def kv_append(k_new, v_new, k_pool, v_pool, page_table, seq_lens, page_size):
    """Pools after appending each sequence's new token, float64 copies.

    "拆开 LLM（二）", section "KV cache": the new token's key and value are
    appended to the cache before it attends. seq_lens[b] counts that token,
    so it becomes logical token n-1 (n = seq_lens[b]) of sequence b: slot
    (n-1) % page_size of physical page page_table[first_b + (n-1) //
    page_size] ("LLM 核心技术", PagedAttention section), every head at once.
    """
    k_out = np.array(k_pool, dtype=np.float64, copy=True)
    v_out = np.array(v_pool, dtype=np.float64, copy=True)
    layout = sequence_pages(seq_lens, page_size)
    for b, n in enumerate(seq_lens):
        t = int(n) - 1
        first, _ = layout[b]
        page = int(page_table[first + t // page_size])
        k_out[page, :, t % page_size, :] = k_new[b]
        v_out[page, :, t % page_size, :] = v_new[b]
    return k_out, v_out


def attention_lse(q, k, v, scale, causal=False, window=0, row_chunk=2048):
    """Log-sum-exp of each row's scaled, masked logits, float64 [B, Hq, Sq].

    lse[b, h, i] = log(sum over visible j of exp(scale * q_i . k_j)), the
    second output of the FlashAttention forward ("Attention From Scratch",
    FlashAttention module returning output and lse); softmax weights are
    exp(S - lse). Computed with the row maximum shifted out first, as in the
    stable softmax of "拆开 LLM（二）" (section "数值稳定的 softmax").
    """
    B, Hq, Sq, _ = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    out = np.empty((B, Hq, Sq), dtype=np.float64)
    vis = visible(Sq, Sk, causal, window)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kb = np.asarray(k[b, g], dtype=np.float64)
            for r0 in range(0, Sq, row_chunk):
                r1 = min(Sq, r0 + row_chunk)
                qr = np.asarray(q[b, h, r0:r1], dtype=np.float64)
                s = _scores(qr, kb, scale, vis[r0:r1])
                m = s.max(axis=1, keepdims=True)
                out[b, h, r0:r1] = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


def prefill_paged(q, k_pool, v_pool, page_table, seq_lens, page_size, scale, causal=False, window=0):
    """Attention of the Sq newest tokens of each sequence over its paged
    cache, float64 [B, Hq, Sq, D].

    q: [B, Hq, Sq, D]; the cache of sequence b holds n = seq_lens[b] tokens
    (the Sq new ones included) in pages of a pool ("LLM 核心技术",
    PagedAttention section). The gathered cache is attended as in
    `attention`, query row i at position n - Sq + i (bottom-right).
    """
    B, Hq, Sq, D = q.shape
    out = np.empty((B, Hq, Sq, v_pool.shape[3]), dtype=np.float64)
    for b in range(B):
        kb = gather_sequence(k_pool, page_table, seq_lens, page_size, b)[None]
        vb = gather_sequence(v_pool, page_table, seq_lens, page_size, b)[None]
        out[b] = attention(np.asarray(q[b:b + 1], dtype=np.float64), kb, vb, scale, causal, window)[0]
    return out


def attention_bwd(q, k, v, do, scale, causal=False, window=0, row_chunk=2048):
    """Gradients (dq, dk, dv), float64, of L = sum(do * O) where O is
    `attention(q, k, v, scale, causal, window)`; shapes as q, k, v.

    The pages name the backward pass only through FlashAttention's
    recomputation ("Attention From Scratch", 进阶篇 §5; "LLM 核心技术", section
    底层算子优化：FlashAttention) and the softmax gradient made of p(1 - p)
    terms ("拆开 LLM（二）", section "√d 不是装饰，是保命符"). This is the plain
    chain rule through the definition, per (batch, query head), with
    S = scale * q k^T masked to -inf and P = softmax(S) by rows:

    * dV = P^T dO and dP = dO V^T;
    * dS = P * (dP - rowsum(P * dP)), the softmax Jacobian diag(p) - p p^T
      applied row by row (masked entries have p = 0, hence dS = 0);
    * dQ = scale * dS K and dK = scale * dS^T Q.

    K/V head g is read by the query heads h with h // (Hq // Hkv) == g
    (repeat_interleave on the head axis, "Attention 机制详解" §5.2), so its dK
    and dV are the sums over those heads. ``row_chunk`` only bounds memory:
    rows contribute to dK and dV independently.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    dq = np.zeros((B, Hq, Sq, D), dtype=np.float64)
    dk = np.zeros((B, Hkv, Sk, D), dtype=np.float64)
    dv = np.zeros((B, Hkv, Sk, v.shape[3]), dtype=np.float64)
    vis = visible(Sq, Sk, causal, window)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            kb = np.asarray(k[b, g], dtype=np.float64)
            vb = np.asarray(v[b, g], dtype=np.float64)
            for r0 in range(0, Sq, row_chunk):
                r1 = min(Sq, r0 + row_chunk)
                qr = np.asarray(q[b, h, r0:r1], dtype=np.float64)
                dor = np.asarray(do[b, h, r0:r1], dtype=np.float64)
                p = softmax_rows(_scores(qr, kb, scale, vis[r0:r1]))
                dv[b, g] += p.T @ dor
                dp = dor @ vb.T
                ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
                dq[b, h, r0:r1] = scale * (ds @ kb)
                dk[b, g] += scale * (ds.T @ qr)
    return dq, dk, dv
