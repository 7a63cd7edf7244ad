"""Seeded random sweep of GPU parity against the float64 oracle.

Prefill (bfloat16 and float32), paged decode (plain and windowed) and the
backward pass, over shapes, masks, scales, head groupings and page sizes drawn
from one numpy generator per family, so that mixes no hand-picked case names
(odd group sizes with windows, negative scales with bottom-right causal rows,
tiny pages with long sequences, ...) are still checked. Scales are drawn up to
0.4 in magnitude, where a sharp softmax can return outputs of magnitude 4 and
more whose bf16 rounding alone exceeds 1e-2, so the bf16 outputs are held to
the fixed bar above their own rounding floor (check_bf16_floor); float32 and
gradients use the named cases' bars. Every case prints its parameters before
its GPU step.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import check_bf16_floor, check_f32, check_grad, cuda, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]

GROUPS = [1, 2, 3, 4, 6, 8, 16]   # query heads per K/V head


def _scale(rng, D):
    # the usual 1/sqrt(D) half of the time, else a uniform draw of either sign
    return 1.0 / math.sqrt(D) if rng.random() < 0.5 else float(rng.uniform(-0.4, 0.4))


def _prefill_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 4]))
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 2))
        Sk = int(rng.integers(1, 700))
        Sq = int(rng.integers(1, Sk + 1)) if causal else int(rng.integers(1, 700))
        window = int(rng.integers(1, Sk + 64)) if causal and rng.random() < 0.5 else 0
        cases.append((B, Hkv * G, Hkv, Sq, Sk, D, causal, window, _scale(rng, D), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _prefill_cases(24, 2024))
def test_random_prefill(case):
    B, Hq, Hkv, Sq, Sk, D, causal, window, scale, seed = case
    for dtype in ("bf16", "f32"):
        say(f"random prefill {dtype} {case}")
        q, k, v = inputs.prefill_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed)
        run = attn.fwd if dtype == "bf16" else attn.fwd_f32
        got = run(*cuda(q, k, v), scale=scale, causal=causal, window=window)
        torch.cuda.synchronize()
        want = oracle.attention(f64(q), f64(k), f64(v), scale, causal, window)
        if dtype == "bf16":
            check_bf16_floor(f64(got.cpu()), want, f"bf16 {case}")
        else:
            check_f32(f64(got.cpu()), want, f"f32 {case}")


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice(GROUPS))
        D = int(rng.choice([64, 128]))
        nseq = int(rng.integers(1, 25))
        lens = [int(x) for x in rng.integers(1, 2500, nseq)]
        ps = int(rng.choice([8, 16, 32, 64, 128, 256]))
        window = int(rng.integers(1, 3000)) if rng.random() < 0.5 else 0
        cases.append((lens, Hkv * G, Hkv, D, ps, window, _scale(rng, D), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _decode_cases(24, 4048))
def test_random_decode(case):
    lens, Hq, Hkv, D, ps, window, scale, seed = case
    say(f"random decode {len(lens)} seqs max len {max(lens)} Hq={Hq} Hkv={Hkv} D={D} page={ps} "
        f"window={window} scale={scale:.4f} seed={seed}")
    d = inputs.decode_inputs(len(lens), Hq, Hkv, D, ps, 0, 0, "bf16", seed=seed, seq_lens=lens)
    q, kp, vp, pt, sl = cuda(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"])
    args = (f64(d["q"]), d["k_pool"].float().numpy(), d["v_pool"].float().numpy(), d["page_table"].numpy(),
            d["seq_lens"].numpy(), ps, scale)
    if window:
        got = attn.decode_paged_window(q, kp, vp, pt, sl, window, scale=scale)
        want = oracle.decode_paged_window(*args, window)
    else:
        got = attn.decode_paged(q, kp, vp, pt, sl, scale=scale)
        want = oracle.decode_paged(*args)
    torch.cuda.synchronize()
    check_bf16_floor(f64(got.cpu()), want, f"decode {len(lens)} seqs, window {window}")


def _backward_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3, 4]))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        Sk = int(rng.integers(1, 400))
        Sq = int(rng.integers(1, Sk + 1)) if causal else int(rng.integers(1, 400))
        window = int(rng.integers(1, Sk + 32)) if causal and rng.random() < 0.5 else 0
        cases.append((1, Hkv * G, Hkv, Sq, Sk, D, causal, window, _scale(rng, D), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _backward_cases(12, 8096))
def test_random_backward(case):
    B, Hq, Hkv, Sq, Sk, D, causal, window, scale, seed = case
    say(f"random backward {case}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, Sq, Sk, D, "bf16", seed)
    do = torch.randn((B, Hq, Sq, D), generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = attn.fwd_lse(qd, kd, vd, scale=scale, causal=causal, window=window)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    want = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, causal, window)
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        check_grad(f64(g.cpu()), w, f"{name} {case}")
