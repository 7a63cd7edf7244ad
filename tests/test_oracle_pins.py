"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each pin is chosen so that a plausible slip in ``oracle/`` (a dropped scale, a
wrong mask sign or off-by-one, a transposed operand, the wrong GQA head, a
softmax without the max shift, pages gathered in the wrong order) fails at
least one test here:

* brute force: a scalar pure-Python loop (math.exp / math.fsum) on tiny inputs;
* closed forms: two-key softmax as a logistic function; position probes where
  Q = 0 makes the weights uniform and V holds the bits of the key index, so
  each output is a count of visible keys with a bit set, computed by formula;
* special cases: a single key, causal row 0, window 1, identical keys, scale 0;
* structure of the causal weight matrix printed on "拆开 LLM（二）" (section
  "从对齐机器到 self-attention");
* equivalences the pages state: GQA with Hkv = Hq is MHA, Hkv = 1 is MQA, both
  equal attention over explicitly repeat_interleave'd K/V ("Attention 机制详解"
  §5.2); a paged cache equals the contiguous one ("LLM 核心技术", section
  PagedAttention); one decode step equals the matching row of a full causal
  pass ("拆开 LLM（二）", section "KV cache");
* the causality test of the LLMs-from-scratch article (gsyq.cn, §5): changing
  future inputs leaves earlier outputs unchanged.
"""

import math

import numpy as np
import pytest

import oracle


# ----------------------------------------------------------------------------
# brute force


def _brute(q, k, v, scale, causal, window):
    """Scalar loops over nested lists: q [B][Hq][Sq][D], k/v [B][Hkv][Sk][D]."""
    B, Hq, Sq = len(q), len(q[0]), len(q[0][0])
    Hkv, Sk, D = len(k[0]), len(k[0][0]), len(v[0][0][0])
    group = Hq // Hkv
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            g = h // group
            oh = []
            for i in range(Sq):
                t = i + (Sk - Sq) + 1          # tokens 0 .. t-1 exist at row i
                first = max(0, t - window) if window else 0
                keys = list(range(first, t)) if causal else list(range(Sk))
                logits = [math.fsum(q[b][h][i][c] * k[b][g][j][c] for c in range(D)) * scale
                          for j in keys]
                top = max(logits)
                w = [math.exp(x - top) for x in logits]
                z = math.fsum(w)
                oh.append([math.fsum(w[n] * v[b][g][j][c] for n, j in enumerate(keys)) / z
                           for c in range(D)])
            ob.append(oh)
        out.append(ob)
    return np.array(out)


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, window
    (1, 1, 1, 5, 5, 3, False, 0),
    (2, 2, 1, 4, 6, 4, False, 0),
    (1, 4, 2, 6, 6, 2, True, 0),
    (2, 4, 4, 3, 7, 3, True, 0),      # Sq < Sk: bottom-right causal
    (1, 2, 1, 7, 7, 4, True, 3),      # sliding window
    (1, 4, 1, 8, 8, 2, True, 1),      # window of one key
    (2, 2, 2, 2, 8, 3, True, 4),      # window with Sq < Sk
    (1, 3, 3, 6, 6, 4, True, 9),      # window wider than the sequence
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force(case):
    B, Hq, Hkv, Sq, Sk, D, causal, window = case
    rng = np.random.default_rng(sum(case[:6]))
    q = rng.standard_normal((B, Hq, Sq, D))
    k = rng.standard_normal((B, Hkv, Sk, D))
    v = rng.standard_normal((B, Hkv, Sk, D))
    scale = 0.7
    want = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal, window)
    got = oracle.attention(q, k, v, scale, causal, window)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# closed forms


def test_two_keys_is_logistic_even_when_exp_would_overflow():
    # softmax over two logits a, b is (sigma(a - b), sigma(b - a)); with logits
    # near 1000, exp without the max shift overflows to inf and gives NaN.
    q = np.array([[[[1.0, 2.0]]]])
    k = np.array([[[[300.0, 250.0], [310.0, 244.0]]]])
    v = np.array([[[[1.0, -3.0], [5.0, 7.0]]]])
    scale = 1.25
    a = scale * (300.0 + 500.0)
    b = scale * (310.0 + 488.0)
    p0 = 1.0 / (1.0 + math.exp(b - a))
    want = p0 * v[0, 0, 0] + (1.0 - p0) * v[0, 0, 1]
    got = oracle.attention(q, k, v, scale)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got[0, 0, 0], want, rtol=0, atol=1e-12)


def _count_bit_below(n, c):
    """#{0 <= j < n : bit c of j is 1}: full periods of 2^(c+1) plus the tail."""
    period = 1 << (c + 1)
    return (n // period) * (1 << c) + max(0, n % period - (1 << c))


def _probe_expected(Sq, Sk, causal, window, nbits):
    """O[i, c] for Q = 0 and V[j, c] = bit c of j, by counting."""
    out = np.zeros((Sq, nbits))
    for i in range(Sq):
        t = i + (Sk - Sq) + 1 if causal else Sk
        first = max(0, t - window) if window else 0
        for c in range(nbits):
            ones = _count_bit_below(t, c) - _count_bit_below(first, c)
            out[i, c] = ones / (t - first)
    return out


@pytest.mark.parametrize("Sq,Sk,causal,window", [
    (37, 37, False, 0), (37, 37, True, 0), (20, 45, True, 0),
    (64, 64, True, 5), (30, 70, True, 16), (50, 50, True, 1), (50, 50, True, 200),
])
def test_position_probe(Sq, Sk, causal, window):
    nbits = 7
    q = np.zeros((1, 1, Sq, nbits))
    k = np.random.default_rng(1).standard_normal((1, 1, Sk, nbits))
    j = np.arange(Sk)
    v = ((j[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.float64)[None, None]
    got = oracle.attention(q, k, v, 0.3, causal, window)[0, 0]
    np.testing.assert_allclose(got, _probe_expected(Sq, Sk, causal, window, nbits), atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (6, 3)])
def test_gqa_head_mapping_probe(Hq, Hkv):
    # V's last column holds the K/V head index, so it comes out unchanged for
    # every query row; the expected head follows repeat_interleave order.
    rng = np.random.default_rng(2)
    S, D = 9, 4
    q = rng.standard_normal((1, Hq, S, D))
    k = rng.standard_normal((1, Hkv, S, D))
    v = rng.standard_normal((1, Hkv, S, D))
    v[..., -1] = np.arange(Hkv)[None, :, None]
    order = np.repeat(np.arange(Hkv), Hq // Hkv)
    got = oracle.attention(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(got[0, :, :, -1], np.broadcast_to(order[:, None], (Hq, S)), atol=1e-12)


# ----------------------------------------------------------------------------
# special cases


def test_special_cases():
    rng = np.random.default_rng(3)
    S, D = 12, 5
    q = rng.standard_normal((1, 1, S, D))
    k = rng.standard_normal((1, 1, S, D))
    v = rng.standard_normal((1, 1, S, D))
    # one key: the output is that key's value
    got = oracle.attention(q, k[:, :, :1], v[:, :, :1], 0.9)
    np.testing.assert_allclose(got[0, 0], np.broadcast_to(v[0, 0, 0], (S, D)), atol=1e-12)
    # causal row 0 sees only key 0
    got = oracle.attention(q, k, v, 0.9, causal=True)
    np.testing.assert_array_equal(got[0, 0, 0], v[0, 0, 0])
    # a window of one key returns V row by row
    got = oracle.attention(q, k, v, 0.9, causal=True, window=1)
    np.testing.assert_array_equal(got[0, 0], v[0, 0])
    # identical keys, scale 0 and Q = 0 all give the mean of the visible values
    want = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    same_k = np.broadcast_to(k[:, :, :1], k.shape)
    for got in (oracle.attention(q, same_k, v, 0.9, causal=True),
                oracle.attention(q, k, v, 0.0, causal=True),
                oracle.attention(np.zeros_like(q), k, v, 0.9, causal=True)):
        np.testing.assert_allclose(got[0, 0], want, atol=1e-12)


def test_softmax_rows_definition():
    x = np.array([[0.0, -np.inf, 1.0], [1000.0, 999.0, -np.inf]])
    p = oracle.softmax_rows(x)
    assert p[0, 1] == 0.0 and p[1, 2] == 0.0
    e = math.e
    np.testing.assert_allclose(p[0], [1 / (1 + e), 0.0, e / (1 + e)], atol=1e-15)
    np.testing.assert_allclose(p[1], [e / (1 + e), 1 / (1 + e), 0.0], atol=1e-15)


def test_weight_matrix_structure_matches_printed_example():
    path = __file__.replace("test_oracle_pins.py", "golden/p5_causal_weights_6x6.txt")
    printed = np.loadtxt(path, comments="#")
    assert printed.shape == (6, 6)
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    w = oracle.attention_weights(q, k, 1 / math.sqrt(8), causal=True)
    np.testing.assert_array_equal(w == 0.0, printed == 0.0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(printed.sum(axis=1), 1.0, atol=0.015)
    # masking with 0 instead of -inf, or after the softmax, breaks one of these
    assert np.all(w[np.tril_indices(6)] > 0)


# ----------------------------------------------------------------------------
# equivalences


def test_gqa_equals_mha_and_mqa_on_repeated_kv():
    rng = np.random.default_rng(5)
    B, Hq, S, D = 2, 6, 10, 4
    q = rng.standard_normal((B, Hq, S, D))
    for Hkv in (6, 3, 2, 1):
        k = rng.standard_normal((B, Hkv, S, D))
        v = rng.standard_normal((B, Hkv, S, D))
        rep = Hq // Hkv
        kk, vv = np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1)
        np.testing.assert_allclose(oracle.attention(q, k, v, 0.4, causal=True),
                                   oracle.attention(q, kk, vv, 0.4, causal=True), atol=1e-13)


def test_rows_and_chunks_match_full():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 4, 33, 8))
    k = rng.standard_normal((2, 2, 40, 8))
    v = rng.standard_normal((2, 2, 40, 8))
    full = oracle.attention(q, k, v, 0.3, causal=True, window=9)
    np.testing.assert_allclose(oracle.attention(q, k, v, 0.3, causal=True, window=9, row_chunk=5),
                               full, atol=1e-14)
    rows = [0, 7, 32, 15]
    np.testing.assert_allclose(oracle.attention_rows(q, k, v, 1, 3, rows, 0.3, True, 9),
                               full[1, 3, rows], atol=1e-14)


def test_bottom_right_alignment_matches_square_pass():
    rng = np.random.default_rng(7)
    S, m, D = 20, 6, 5
    q = rng.standard_normal((1, 2, S, D))
    k = rng.standard_normal((1, 1, S, D))
    v = rng.standard_normal((1, 1, S, D))
    for window in (0, 4):
        full = oracle.attention(q, k, v, 0.8, causal=True, window=window)
        tail = oracle.attention(q[:, :, S - m:], k, v, 0.8, causal=True, window=window)
        np.testing.assert_allclose(tail, full[:, :, S - m:], atol=1e-14)


def _paged_from_contiguous(kc, vc, lens, page_size, rng, permute):
    """Scatter contiguous [B, Hkv, Smax, D] caches into a shuffled page pool."""
    counts = [(n + page_size - 1) // page_size for n in lens]
    total = sum(counts)
    perm = rng.permutation(total) if permute else np.arange(total)
    Hkv, D = kc.shape[1], kc.shape[3]
    kp = np.full((total, Hkv, page_size, D), np.nan)
    vp = np.full((total, Hkv, page_size, D), np.nan)
    entry = 0
    for b, n in enumerate(lens):
        for t in range(n):
            page = perm[entry + t // page_size]
            kp[page, :, t % page_size] = kc[b, :, t]
            vp[page, :, t % page_size] = vc[b, :, t]
        entry += counts[b]
    return kp, vp, perm.astype(np.int32)


@pytest.mark.parametrize("permute", [False, True])
def test_paged_equals_contiguous(permute):
    rng = np.random.default_rng(8)
    lens = [1, 16, 17, 40, 5]
    B, Hq, Hkv, D, ps = len(lens), 4, 2, 6, 8
    Smax = max(lens)
    kc = rng.standard_normal((B, Hkv, Smax, D))
    vc = rng.standard_normal((B, Hkv, Smax, D))
    q = rng.standard_normal((B, Hq, D))
    kp, vp, table = _paged_from_contiguous(kc, vc, lens, ps, rng, permute)
    got = oracle.decode_paged(q, kp, vp, table, np.array(lens), ps, 0.6)
    assert np.all(np.isfinite(got))  # NaN padding is never read
    for b, n in enumerate(lens):
        want = oracle.attention(q[b][None, :, None, :], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], 0.6)
        np.testing.assert_allclose(got[b], want[0, :, 0, :], atol=1e-13)


def test_paged_position_probe():
    # V slot of logical token t holds the bits of t; Q = 0 -> mean of bits.
    rng = np.random.default_rng(9)
    lens, ps, nbits = [3, 16, 33, 100], 16, 7
    B, Hkv = len(lens), 2
    Smax = max(lens)
    kc = rng.standard_normal((B, Hkv, Smax, nbits))
    bits = ((np.arange(Smax)[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.float64)
    vc = np.broadcast_to(bits, (B, Hkv, Smax, nbits)).copy()
    kp, vp, table = _paged_from_contiguous(kc, vc, lens, ps, rng, True)
    got = oracle.decode_paged(np.zeros((B, 4, nbits)), kp, vp, table, np.array(lens), ps, 1.0)
    for b, n in enumerate(lens):
        want = [_count_bit_below(n, c) / n for c in range(nbits)]
        np.testing.assert_allclose(got[b], np.broadcast_to(want, (4, nbits)), atol=1e-12)


def test_incremental_decode_equals_full_recompute():
    rng = np.random.default_rng(10)
    n, Hq, Hkv, D, ps = 21, 4, 2, 5, 4
    q = rng.standard_normal((1, Hq, n, D))
    k = rng.standard_normal((1, Hkv, n, D))
    v = rng.standard_normal((1, Hkv, n, D))
    full = oracle.attention(q, k, v, 0.5, causal=True)
    for t in range(1, n + 1):
        kp, vp, table = _paged_from_contiguous(k, v, [t], ps, rng, True)
        step = oracle.decode_paged(q[:, :, t - 1], kp, vp, table, np.array([t]), ps, 0.5)
        np.testing.assert_allclose(step[0], full[0, :, t - 1], atol=1e-13)


@pytest.mark.parametrize("window", [0, 3])
def test_future_perturbation_leaves_past_rows_unchanged(window):
    # gsyq.cn article §5: add 10 to every input after position 2; the outputs
    # of the first positions must not move. Here K and V after (and, with a
    # window, long before) each probed row are perturbed.
    rng = np.random.default_rng(11)
    S, D = 12, 6
    q = rng.standard_normal((1, 3, S, D))
    k = rng.standard_normal((1, 3, S, D))
    v = rng.standard_normal((1, 3, S, D))
    base = oracle.attention(q, k, v, 0.5, causal=True, window=window)
    for i in (0, 2, 7):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] += 10.0
        v2[:, :, i + 1:] += 10.0
        if window:
            k2[:, :, :max(0, i - window + 1)] -= 10.0
            v2[:, :, :max(0, i - window + 1)] -= 10.0
        pert = oracle.attention(q, k2, v2, 0.5, causal=True, window=window)
        np.testing.assert_array_equal(pert[:, :, i], base[:, :, i])


def test_visible_rejects_window_without_causal():
    with pytest.raises(ValueError):
        oracle.visible(4, 4, causal=False, window=2)


def test_sequence_pages_layout():
    assert oracle.sequence_pages([1, 16, 17, 32], 16) == [(0, 1), (1, 1), (2, 2), (4, 2)]


# ----------------------------------------------------------------------------
# sliding-window decode


@pytest.mark.parametrize("window", [1, 3, 8, 16, 50])
def test_window_decode_matches_brute_force(window):
    # the new token at position n-1 sees positions max(0, n-window) .. n-1
    rng = np.random.default_rng(12)
    lens = [1, 5, 9, 16, 23]
    B, Hq, Hkv, D, ps = len(lens), 4, 2, 3, 8
    Smax = max(lens)
    kc = rng.standard_normal((B, Hkv, Smax, D))
    vc = rng.standard_normal((B, Hkv, Smax, D))
    q = rng.standard_normal((B, Hq, D))
    kp, vp, table = _paged_from_contiguous(kc, vc, lens, ps, rng, True)
    got = oracle.decode_paged_window(q, kp, vp, table, np.array(lens), ps, 0.7, window)
    for b, n in enumerate(lens):
        want = _brute(q[b:b + 1, :, None, :].tolist(), kc[b:b + 1, :, :n].tolist(),
                      vc[b:b + 1, :, :n].tolist(), 0.7, True, window)
        np.testing.assert_allclose(got[b], want[0, :, 0, :], atol=1e-12)


def test_window_decode_position_probe():
    # Q = 0 -> mean over the window of the bits of the token index
    rng = np.random.default_rng(13)
    lens, ps, nbits, W = [3, 16, 33, 100], 16, 7, 20
    B, Hkv = len(lens), 2
    Smax = max(lens)
    kc = rng.standard_normal((B, Hkv, Smax, nbits))
    bits = ((np.arange(Smax)[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.float64)
    vc = np.broadcast_to(bits, (B, Hkv, Smax, nbits)).copy()
    kp, vp, table = _paged_from_contiguous(kc, vc, lens, ps, rng, True)
    got = oracle.decode_paged_window(np.zeros((B, 4, nbits)), kp, vp, table, np.array(lens), ps, 1.0, W)
    for b, n in enumerate(lens):
        lo = max(0, n - W)
        want = [(_count_bit_below(n, c) - _count_bit_below(lo, c)) / (n - lo) for c in range(nbits)]
        np.testing.assert_allclose(got[b], np.broadcast_to(want, (4, nbits)), atol=1e-12)


def test_window_decode_special_cases():
    rng = np.random.default_rng(14)
    lens = [1, 7, 30]
    B, Hq, Hkv, D, ps = len(lens), 2, 1, 5, 8
    Smax = max(lens)
    kc = rng.standard_normal((B, Hkv, Smax, D))
    vc = rng.standard_normal((B, Hkv, Smax, D))
    q = rng.standard_normal((B, Hq, D))
    kp, vp, table = _paged_from_contiguous(kc, vc, lens, ps, rng, True)
    sl = np.array(lens)
    full = oracle.decode_paged(q, kp, vp, table, sl, ps, 0.4)
    # no window, or a window at least as long as every sequence: plain decode
    for W in (0, 30, 1000):
        np.testing.assert_allclose(oracle.decode_paged_window(q, kp, vp, table, sl, ps, 0.4, W), full, atol=1e-14)
    # a window of one token returns that token's V row
    one = oracle.decode_paged_window(q, kp, vp, table, sl, ps, 0.4, 1)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(one[b], np.broadcast_to(vc[b, 0, n - 1], (Hq, D)), atol=1e-15)


# ----------------------------------------------------------------------------
# KV append


def test_append_then_gather_is_the_longer_cache():
    rng = np.random.default_rng(15)
    lens = [1, 8, 9, 30]               # lengths after the append
    B, Hkv, D, ps = len(lens), 2, 3, 8
    Smax = max(lens)
    kc = rng.standard_normal((B, Hkv, Smax, D))
    vc = rng.standard_normal((B, Hkv, Smax, D))
    kp, vp, table = _paged_from_contiguous(kc, vc, lens, ps, rng, True)
    # wipe the last token of each sequence, then append it back
    kn = np.stack([kc[b, :, n - 1] for b, n in enumerate(lens)])
    vn = np.stack([vc[b, :, n - 1] for b, n in enumerate(lens)])
    layout = oracle.sequence_pages(lens, ps)
    for b, n in enumerate(lens):
        page = table[layout[b][0] + (n - 1) // ps]
        kp[page, :, (n - 1) % ps] = 0.0
        vp[page, :, (n - 1) % ps] = 0.0
    k2, v2 = oracle.kv_append(kn, vn, kp, vp, table, lens, ps)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(oracle.gather_sequence(k2, table, lens, ps, b), kc[b, :, :n])
        np.testing.assert_array_equal(oracle.gather_sequence(v2, table, lens, ps, b), vc[b, :, :n])
    # nothing else moved: only one slot per sequence differs from the input
    same = (k2 == kp) | (np.isnan(k2) & np.isnan(kp))     # NaN padding compares equal
    changed = np.argwhere(np.any(~same, axis=(1, 3)))     # (page, slot) pairs
    assert len(changed) == len(lens)


def test_append_and_decode_step_by_step_equals_causal_prefill():
    # start from an empty cache, append one token per step, decode it
    rng = np.random.default_rng(16)
    n, Hq, Hkv, D, ps = 19, 4, 2, 5, 4
    q = rng.standard_normal((1, Hq, n, D))
    k = rng.standard_normal((1, Hkv, n, D))
    v = rng.standard_normal((1, Hkv, n, D))
    full = oracle.attention(q, k, v, 0.5, causal=True)
    pages = rng.permutation(8)         # pool of 8 pages handed out in this order
    kp = np.full((8, Hkv, ps, D), np.nan)
    vp = np.full((8, Hkv, ps, D), np.nan)
    for t in range(1, n + 1):
        table = pages[:(t + ps - 1) // ps].astype(np.int32)
        kp, vp = oracle.kv_append(k[:, :, t - 1], v[:, :, t - 1], kp, vp, table, [t], ps)
        step = oracle.decode_paged(q[:, :, t - 1], kp, vp, table, np.array([t]), ps, 0.5)
        np.testing.assert_allclose(step[0], full[0, :, t - 1], atol=1e-13)


# ----------------------------------------------------------------------------
# log-sum-exp


def _brute_lse(q, k, scale, causal, window):
    B, Hq, Sq = len(q), len(q[0]), len(q[0][0])
    Hkv, Sk, D = len(k[0]), len(k[0][0]), len(k[0][0][0])
    out = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Sq):
                t = i + (Sk - Sq) + 1
                first = max(0, t - window) if window else 0
                keys = list(range(first, t)) if causal else list(range(Sk))
                out[b, h, i] = math.log(math.fsum(
                    math.exp(math.fsum(q[b][h][i][c] * k[b][g][j][c] for c in range(D)) * scale) for j in keys))
    return out


@pytest.mark.parametrize("case", CASES)
def test_lse_brute_force(case):
    B, Hq, Hkv, Sq, Sk, D, causal, window = case
    rng = np.random.default_rng(sum(case[:6]))
    q = rng.standard_normal((B, Hq, Sq, D))
    k = rng.standard_normal((B, Hkv, Sk, D))
    v = rng.standard_normal((B, Hkv, Sk, D))
    got = oracle.attention_lse(q, k, v, 0.7, causal, window)
    np.testing.assert_allclose(got, _brute_lse(q.tolist(), k.tolist(), 0.7, causal, window), atol=1e-12)


def test_lse_closed_forms():
    rng = np.random.default_rng(17)
    S, D = 9, 4
    k = rng.standard_normal((1, 1, S, D))
    v = rng.standard_normal((1, 1, S, D))
    # Q = 0: every visible logit is 0, lse = log(number of visible keys)
    lse = oracle.attention_lse(np.zeros((1, 1, S, D)), k, v, 1.0, causal=True, window=4)
    np.testing.assert_allclose(lse[0, 0], np.log([min(i + 1, 4) for i in range(S)]), atol=1e-15)
    # softmax weights are exp(S - lse): rows of the weight matrix
    q = rng.standard_normal((1, 1, S, D))
    w = oracle.attention_weights(q[0, 0], k[0, 0], 0.3, causal=True)
    lse = oracle.attention_lse(q, k, v, 0.3, causal=True)[0, 0]
    s = q[0, 0] @ k[0, 0].T * 0.3
    vis = oracle.visible(S, S, True, 0)
    np.testing.assert_allclose(np.where(vis, np.exp(s - lse[:, None]), 0.0), w, atol=1e-14)
    # huge logits do not overflow: two keys with logits 1000 and 1000 - d
    q2 = np.array([[[[1000.0]]]])
    k2 = np.array([[[[1.0], [0.99]]]])
    lse2 = oracle.attention_lse(q2, k2, k2, 1.0)
    np.testing.assert_allclose(lse2[0, 0, 0], 1000.0 + math.log1p(math.exp(-10.0)), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# prefill against a paged cache


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 5)])
def test_paged_prefill_matches_brute_force_and_decode(causal, window):
    rng = np.random.default_rng(18)
    lens = [7, 16, 20]
    B, Hq, Hkv, Sq, D, ps = len(lens), 4, 2, 3, 3, 8
    Smax = max(lens)
    kc = rng.standard_normal((B, Hkv, Smax, D))
    vc = rng.standard_normal((B, Hkv, Smax, D))
    q = rng.standard_normal((B, Hq, Sq, D))
    kp, vp, table = _paged_from_contiguous(kc, vc, lens, ps, rng, True)
    got = oracle.prefill_paged(q, kp, vp, table, np.array(lens), ps, 0.6, causal, window)
    for b, n in enumerate(lens):
        want = _brute(q[b:b + 1].tolist(), kc[b:b + 1, :, :n].tolist(), vc[b:b + 1, :, :n].tolist(), 0.6,
                      causal, window)
        np.testing.assert_allclose(got[b], want[0], atol=1e-12)
    if causal:
        # the last query row is the decode step of the last token
        last = oracle.decode_paged_window(q[:, :, -1], kp, vp, table, np.array(lens), ps, 0.6, window)
        np.testing.assert_allclose(got[:, :, -1], last, atol=1e-13)


# ----------------------------------------------------------------------------
# backward pass: gradients of L = sum(dO * O)


def _loss_brute(q, k, v, do, scale, causal, window):
    return float(np.sum(do * _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal, window)))


def _fd_grads(q, k, v, do, scale, causal, window, h=1e-5):
    """Central differences of the brute-force forward, element by element."""
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[idx]
            x[idx] = keep + h
            up = _loss_brute(q, k, v, do, scale, causal, window)
            x[idx] = keep - h
            dn = _loss_brute(q, k, v, do, scale, causal, window)
            x[idx] = keep
            g[idx] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


def _bwd_inputs(case, seed_extra=0):
    B, Hq, Hkv, Sq, Sk, D, causal, window = case
    rng = np.random.default_rng(sum(case[:6]) + 100 + seed_extra)
    q = rng.standard_normal((B, Hq, Sq, D))
    k = rng.standard_normal((B, Hkv, Sk, D))
    v = rng.standard_normal((B, Hkv, Sk, D))
    do = rng.standard_normal((B, Hq, Sq, D))
    return q, k, v, do


@pytest.mark.parametrize("case", CASES)
def test_bwd_matches_finite_differences_of_brute_force(case):
    causal, window = case[6], case[7]
    q, k, v, do = _bwd_inputs(case)
    scale = 0.7
    want = _fd_grads(q, k, v, do, scale, causal, window)
    got = oracle.attention_bwd(q, k, v, do, scale, causal, window)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=0, atol=2e-7)


def test_bwd_pins_reject_plausible_slips():
    # the finite-difference pin fails for each of these variants of the chain
    # rule, computed here beside the oracle's arithmetic
    case = (1, 2, 1, 5, 6, 3, True, 0)
    q, k, v, do = _bwd_inputs(case)
    scale = 0.7
    fd = _fd_grads(q, k, v, do, scale, True, 0)
    vis = oracle.visible(5, 6, True, 0)

    def grads(variant):
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for hq in range(2):
            p = oracle.attention_weights(q[0, hq], k[0, 0], scale, True)
            dp = do[0, hq] @ v[0, 0].T
            rs = np.sum(p * dp, axis=1, keepdims=True)
            ds = p * dp if variant == "no_rowsum" else p * (dp - rs)
            if variant == "mask_after":  # Jacobian applied as if masked keys had weight
                ds = np.where(vis, ds, dp)
            s = 1.0 if variant == "no_scale" else scale
            dk[0, 0] += s * ds.T @ q[0, hq]
            dq[0, hq] = s * ds @ (v[0, 0] if variant == "dq_from_v" else k[0, 0])
            dv[0, 0] += (dp if variant == "dv_from_dp" else p).T @ do[0, hq]
        return dq, dk, dv

    def close(gs):
        return all(np.allclose(g, w, rtol=0, atol=2e-7) for g, w in zip(gs, fd))

    assert close(oracle.attention_bwd(q, k, v, do, scale, True, 0))
    assert close(grads("none"))
    for variant in ("no_rowsum", "mask_after", "no_scale", "dv_from_dp", "dq_from_v"):
        assert not close(grads(variant)), variant


def test_bwd_two_keys_closed_form():
    # one query, two keys: O = s v0 + (1 - s) v1 with s = sigma(z),
    # z = scale q . (k0 - k1); dO . dO/dz = s (1 - s) dO . (v0 - v1), the
    # p (1 - p) factor of the softmax gradient
    q = np.array([[[[0.3, -1.2, 0.5]]]])
    k = np.array([[[[1.0, 0.4, -0.7], [-0.2, 0.9, 0.1]]]])
    v = np.array([[[[2.0, -1.0, 0.5], [0.25, 3.0, -2.0]]]])
    do = np.array([[[[0.7, -0.4, 1.1]]]])
    scale = 0.9
    z = scale * float(q[0, 0, 0] @ (k[0, 0, 0] - k[0, 0, 1]))
    s = 1.0 / (1.0 + math.exp(-z))
    t = s * (1.0 - s) * float(do[0, 0, 0] @ (v[0, 0, 0] - v[0, 0, 1]))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale)
    np.testing.assert_allclose(dq[0, 0, 0], scale * t * (k[0, 0, 0] - k[0, 0, 1]), atol=1e-14)
    np.testing.assert_allclose(dk[0, 0, 0], scale * t * q[0, 0, 0], atol=1e-14)
    np.testing.assert_allclose(dk[0, 0, 1], -scale * t * q[0, 0, 0], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0, 0], s * do[0, 0, 0], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0, 1], (1.0 - s) * do[0, 0, 0], atol=1e-14)


def test_bwd_special_cases():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, S, D = 2, 4, 2, 6, 3
    q = rng.standard_normal((B, Hq, S, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    do = rng.standard_normal((B, Hq, S, D))
    group_sum = do.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=2)
    # a single key: O = V[0] for every row, nothing depends on q or k
    dq, dk, dv = oracle.attention_bwd(q, k[:, :, :1], v[:, :, :1], do, 0.8)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[:, :, 0], group_sum.sum(axis=2), atol=1e-13)
    # window 1: O = V, the same
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.8, causal=True, window=1)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv, group_sum, atol=1e-13)
    # scale 0: uniform weights over the visible keys, no gradient to q or k
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.0, causal=True)
    assert np.all(dq == 0) and np.all(dk == 0)
    want = np.zeros_like(v)
    for i in range(S):
        want[:, :, : i + 1] += group_sum[:, :, i : i + 1] / (i + 1)
    np.testing.assert_allclose(dv, want, atol=1e-13)


@pytest.mark.parametrize("case", CASES)
def test_bwd_invariants(case):
    B, Hq, Hkv, Sq, Sk, D, causal, window = case
    q, k, v, do = _bwd_inputs(case, seed_extra=7)
    scale = 0.45
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal, window)
    o = oracle.attention(q, k, v, scale, causal, window)
    G = Hq // Hkv
    # adding one vector to every key shifts each row's logits by a constant,
    # which the softmax ignores: the key gradients of a head sum to zero
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # logits depend on q and k only through scale * q k^T: scaling q and
    # scaling k act alike, so sum(dq * q) = sum(dk * k) per K/V head
    lhs = (dq * q).reshape(B, Hkv, G, Sq, D).sum(axis=(2, 3, 4))
    rhs = (dk * k).sum(axis=(2, 3))
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    # O is linear in V: sum(dv * v) = L = sum(do * O)
    np.testing.assert_allclose((dv * v).sum(), (do * o).sum(), atol=1e-12)
