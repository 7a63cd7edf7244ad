"""GPU parity of attn_bwd against the float64 oracle's gradients.

The GPU side runs the product pipeline: attn_fwd_lse gives o and lse, then
attn_bwd turns (q, k, v, o, do, lse) into (dq, dk, dv). The oracle computes
its gradients from q, k, v, do alone (its own softmax, no GPU value), on the
same seeded bf16 inputs. Tolerance (tests/gpu_util.py): per element
|err| <= 0.15 (|want| + rms(want)), mean |err| <= 0.005 rms(want), sized from
a CPU emulation of the kernels' bf16 roundings. The full-size workload is
checked on whole K/V head groups the oracle computes slice by slice, in the
launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import check_grad, cuda, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _gpu_bwd(q, k, v, do, scale, causal, window):
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = attn.fwd_lse(qd, kd, vd, scale=scale, causal=causal, window=window)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, window
    (1, 4, 2, 300, 300, 128, True, 0),        # ragged tails, GQA
    (2, 4, 4, 200, 333, 64, False, 0),        # full attention, Sq != Sk, D = 64
    (1, 4, 1, 513, 777, 128, True, 0),        # bottom-right causal, MQA
    (1, 2, 1, 600, 600, 128, True, 100),      # sliding window
    (1, 2, 2, 257, 1000, 128, True, 130),     # window, Sq < Sk: early keys seen by no query
    (2, 6, 3, 256, 256, 64, True, 0),         # D = 64 causal GQA
    (1, 2, 1, 130, 130, 128, True, 1),        # window of one key
    (1, 4, 2, 1, 500, 128, True, 0),          # one query row (a decode step)
    (1, 8, 2, 1024, 1024, 128, True, 0),      # several workgroups per head
    (1, 2, 1, 64, 64, 128, False, 0),         # one tile
    (1, 4, 2, 100, 700, 64, True, 50),        # D = 64 window
    (1, 2, 1, 300, 100, 64, False, 0),        # full attention with Sq > Sk
    (1, 8, 1, 200, 200, 128, True, 0),        # eight query heads on one K/V head
    (2, 4, 2, 65, 65, 128, True, 17),         # one tile plus one row, window
    (1, 2, 2, 600, 300, 128, False, 0),       # full attention, more queries than keys, MHA
    (1, 8, 1, 1500, 1500, 64, True, 0),       # MQA: key blocks split into runs, partials summed
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_oracle(case):
    B, Hq, Hkv, Sq, Sk, D, causal, window = case
    say(f"backward B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} window={window}")
    q, k, v, do = inputs.backward_inputs(B, Hq, Hkv, Sq, Sk, D, seed=sum(case[:6]))
    scale = 1.0 / math.sqrt(D)
    got = _gpu_bwd(q, k, v, do, scale, causal, window)
    want = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, causal, window)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        check_grad(f64(g), w, name)


@pytest.mark.parametrize("scale", [-0.07, 0.0, 0.4])
def test_backward_unusual_scales(scale):
    # a negative scale flips which logit is largest; scale 0 gives uniform
    # weights and zero dq, dk; a large one gives peaked weights
    B, Hq, Hkv, S, D = 1, 2, 1, 200, 128
    say(f"backward scale={scale}")
    q, k, v, do = inputs.backward_inputs(B, Hq, Hkv, S, S, D, seed=77)
    got = _gpu_bwd(q, k, v, do, scale, True, 0)
    want = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, True, 0)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        if scale == 0.0 and name != "dv":
            assert torch.count_nonzero(g) == 0, name
        else:
            check_grad(f64(g), w, name)


def test_backward_without_query_rows_zeroes_dk_dv():
    say("backward Sq=0")
    k = torch.randn(1, 2, 96, 128).to(torch.bfloat16).cuda()
    q = torch.empty(1, 4, 0, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 4, 0, dtype=torch.float32, device="cuda")
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    attn.bwd(q, k, k, q, q, lse, causal=False, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0


def test_backward_is_deterministic():
    # dk, dv are plain stores or a fixed-order sum of split partials (this
    # shape is split) and dq one workgroup's sum: repeated calls agree bit for bit
    say("backward determinism")
    q, k, v, do = cuda(*inputs.backward_inputs(1, 4, 2, 700, 700, 128, seed=5))
    o, lse = attn.fwd_lse(q, k, v, causal=True)
    first = attn.bwd(q, k, v, o, do, lse, causal=True)
    second = attn.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)


def test_full_size_workload_head_groups():
    name = "gqa_causal_4k_bwd"
    w = inputs.WORKLOADS[name]
    say(f"backward workload {name}")
    q, k, v, do = inputs.workload_inputs(name)
    scale = 1.0 / math.sqrt(w["D"])
    dq, dk, dv = _gpu_bwd(q, k, v, do, scale, w["causal"], w["window"])
    G = w["Hq"] // w["Hkv"]
    for b, g in [(0, 0), (w["B"] - 1, w["Hkv"] - 1), (2, 5)]:
        say(f"  oracle on batch {b}, kv head {g}")
        hs = slice(g * G, (g + 1) * G)
        want = oracle.attention_bwd(f64(q[b:b + 1, hs]), f64(k[b:b + 1, g:g + 1]), f64(v[b:b + 1, g:g + 1]),
                                    f64(do[b:b + 1, hs]), scale, w["causal"], w["window"], row_chunk=1024)
        check_grad(f64(dq[b:b + 1, hs]), want[0], f"dq b={b} g={g}")
        check_grad(f64(dk[b:b + 1, g:g + 1]), want[1], f"dk b={b} g={g}")
        check_grad(f64(dv[b:b + 1, g:g + 1]), want[2], f"dv b={b} g={g}")


def test_weight_ordered_rounds_head_groups():
    # more dQ items (128-row query tiles) than workgroup slots, in groups of
    # one head: each XCD takes its items heaviest query tile first
    B, Hq, Hkv, S, D = 4, 16, 16, 2048, 128
    say(f"backward weight-ordered rounds B={B} Hq={Hq} S={S} D={D}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, S, D, "bf16", 62)
    do = torch.randn((B, Hq, S, D), generator=torch.Generator().manual_seed(63)).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = attn.fwd_lse(qd, kd, vd, scale=scale, causal=True)
    # outputs start as NaN: an item that no workgroup took leaves them so
    outs = [torch.full_like(t, float("nan")) for t in (qd, kd, vd)]
    attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=True, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu() for t in outs)
    assert all(torch.isfinite(t.float()).all() for t in (dq, dk, dv))
    for b, h in [(0, 0), (B - 1, Hq - 1), (2, 7)]:
        say(f"  oracle on batch {b}, head {h}")
        s = (slice(b, b + 1), slice(h, h + 1))
        want = oracle.attention_bwd(f64(q[s]), f64(k[s]), f64(v[s]), f64(do[s]), scale, True, 0, row_chunk=1024)
        for name, g, w in zip(("dq", "dk", "dv"), (dq[s], dk[s], dv[s]), want):
            check_grad(f64(g), w, f"{name} b={b} h={h}")


def test_paired_key_blocks_d64_odd_count():
    # enough (batch, kv head, 128-key) blocks for one run each, so under a
    # causal mask the dK/dV workgroups take key blocks in pairs: 65 blocks per
    # (batch, kv head) (the middle one alone, the last one 33 keys), Sq < Sk
    # (bottom-right), D = 64; outputs start as NaN so that a block no
    # workgroup took shows up
    B, Hq, Hkv, Sq, Sk, D = 2, 8, 4, 3000, 8225, 64
    say(f"backward paired key blocks B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, Sq, Sk, D, "bf16", 64)
    do = torch.randn((B, Hq, Sq, D), generator=torch.Generator().manual_seed(65)).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = attn.fwd_lse(qd, kd, vd, scale=scale, causal=True)
    outs = [torch.full_like(t, float("nan")) for t in (qd, kd, vd)]
    attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=True, dq=outs[0], dk=outs[1], dv=outs[2])
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu() for t in outs)
    assert all(torch.isfinite(t.float()).all() for t in (dq, dk, dv))
    G = Hq // Hkv
    for b, g in [(0, 0), (B - 1, Hkv - 1)]:
        say(f"  oracle on batch {b}, kv head {g}")
        hs = slice(g * G, (g + 1) * G)
        want = oracle.attention_bwd(f64(q[b:b + 1, hs]), f64(k[b:b + 1, g:g + 1]), f64(v[b:b + 1, g:g + 1]),
                                    f64(do[b:b + 1, hs]), scale, True, 0, row_chunk=1024)
        check_grad(f64(dq[b:b + 1, hs]), want[0], f"dq b={b} g={g}")
        check_grad(f64(dk[b:b + 1, g:g + 1]), want[1], f"dk b={b} g={g}")
        check_grad(f64(dv[b:b + 1, g:g + 1]), want[2], f"dv b={b} g={g}")
