"""Algorithmic work and byte counts used to express throughput (host logic only).

Conventions (pinned in ``tests/test_work_counts.py`` against the pages' tables):

* Attention costs 4·D flop per visible (query, key) pair: 2·D for the q·k dot
  product and 2·D for accumulating p·v. "拆开 LLM（二）：手撕注意力", section
  "KV cache", prints last-step FLOP counts for a 64-dim layer that equal
  6nD² + 4n²D + 2D² without a cache and 8D² + 4nD with one; the attention
  terms are 4·D per pair.
* The backward pass costs 10·D flop per visible pair (``backward_flops``).
* The KV cache holds 2·Hkv·D elements per token and layer (K and V), as in the
  KV-memory formulas of "LLM 核心技术：Attention 机制的实现与优化" (section
  "内存开销对比") and the per-token table of "拆开 LLM（二）" (section
  "代价：显存里躺着一头大象").
"""


def _sum_min(a, b, w):
    """sum(min(w, x) for x in range(a, b + 1)) for 1 <= a <= b."""
    if b <= w:
        return (a + b) * (b - a + 1) // 2
    if a >= w:
        return w * (b - a + 1)
    return (a + w) * (w - a + 1) // 2 + w * (b - w)


def visible_pairs(Sq, Sk, causal, window):
    """Number of visible (query, key) pairs of one head.

    Query row i sits at position p = i + Sk - Sq and sees keys max(0, p-W+1)
    .. p when causal (all of them when not), so row i contributes
    min(W, p + 1) keys with a window and p + 1 without one.
    """
    if Sq <= 0 or Sk <= 0:
        return 0
    if not causal:
        return Sq * Sk
    off = Sk - Sq
    a, b = off + 1, off + Sq
    if window > 0:
        return _sum_min(a, b, window)
    return (a + b) * Sq // 2


def attention_flops(pairs, D):
    """4·D flop per visible pair (q·k and p·v, 2 flop per multiply-add)."""
    return 4 * D * pairs


def prefill_flops(B, Hq, Sq, Sk, D, causal, window):
    return attention_flops(B * Hq * visible_pairs(Sq, Sk, causal, window), D)


def backward_flops(B, Hq, Sq, Sk, D, causal, window):
    """Algorithmic flop of the backward pass: 10·D per visible pair.

    Five products of 2·D flop per pair: the scores recomputed from q and k,
    dP = dO V^T, dV = P^T dO, dQ = dS K and dK = dS^T Q, i.e. 2.5 times the
    forward count. A kernel that recomputes the scores twice does more work
    than this; the count is the method's, not the kernels'.
    """
    return 10 * D * visible_pairs(Sq, Sk, causal, window) * B * Hq


def kv_bytes_per_token(Hkv, D, elem_bytes):
    """K and V bytes one token occupies in one layer's cache."""
    return 2 * Hkv * D * elem_bytes


def decode_kv_bytes(seq_lens, Hkv, D, elem_bytes=2):
    """Bytes of valid K/V a decode step must read: every cached token once."""
    return sum(int(n) for n in seq_lens) * kv_bytes_per_token(Hkv, D, elem_bytes)


def decode_window_kv_bytes(seq_lens, Hkv, D, window, elem_bytes=2):
    """Bytes of valid K/V a windowed decode step must read: the min(len, W)
    most recent tokens of each sequence (W = 0: all of them)."""
    if window <= 0:
        return decode_kv_bytes(seq_lens, Hkv, D, elem_bytes)
    return sum(min(int(n), window) for n in seq_lens) * kv_bytes_per_token(Hkv, D, elem_bytes)
