"""GPU parity of attn_decode_paged and attn_decode_paged_window against the
float64 oracle.

Padding slots of every sequence's last page hold NaN, so any read of a token
at or past seq_lens[b] shows up as a non-finite output.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import check_bf16, cuda, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run(d, scale):
    q, kp, vp, pt, sl = cuda(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"])
    o = attn.decode_paged(q, kp, vp, pt, sl, scale=scale)
    torch.cuda.synchronize()
    return o.cpu()


def _oracle(d, scale):
    return oracle.decode_paged(f64(d["q"]), d["k_pool"].float().numpy(), d["v_pool"].float().numpy(),
                               d["page_table"].numpy(), d["seq_lens"].numpy(), d["k_pool"].shape[2], scale)


def _run_w(d, scale, window):
    q, kp, vp, pt, sl = cuda(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"])
    o = attn.decode_paged_window(q, kp, vp, pt, sl, window, scale=scale)
    torch.cuda.synchronize()
    return o.cpu()


def _oracle_w(d, scale, window):
    return oracle.decode_paged_window(f64(d["q"]), d["k_pool"].float().numpy(), d["v_pool"].float().numpy(),
                                      d["page_table"].numpy(), d["seq_lens"].numpy(), d["k_pool"].shape[2],
                                      scale, window)


def test_paged_decode_workload():
    w = inputs.WORKLOADS["paged_decode"]
    say("decode workload paged_decode")
    d = inputs.workload_inputs("paged_decode")
    scale = 1.0 / math.sqrt(w["D"])
    got = _run(d, scale)
    check_bf16(f64(got), _oracle(d, scale), "paged_decode")


CASES = [
    # nseq, Hq, Hkv, D, page_size, seq_lens
    (1, 1, 1, 128, 16, [1]),
    (3, 4, 4, 64, 8, [1, 8, 9]),
    (4, 8, 2, 128, 16, [15, 16, 17, 33]),
    (5, 32, 8, 128, 16, [500, 1, 64, 63, 1000]),
    (2, 16, 1, 128, 32, [700, 5]),          # MQA, 16 heads per K/V head
    (3, 12, 12, 64, 64, [130, 64, 1]),
    (2, 8, 2, 128, 256, [300, 1000]),
    (2, 6, 2, 64, 128, [129, 2]),           # 3 heads per K/V head
    (64, 4, 2, 128, 16, list(range(1, 65))),
    # eight and more heads per K/V head: the MFMA kernel
    (4, 16, 2, 128, 16, [1, 31, 33, 2000]),
    (3, 32, 2, 64, 8, [700, 65, 5]),
    (2, 48, 1, 128, 32, [900, 40]),         # a group of 32 heads and one of 16
    (2, 64, 1, 64, 256, [1500, 3]),         # MQA, two groups of 32
    (40, 64, 8, 128, 16, [37 * i % 1900 + 1 for i in range(40)]),
]


@pytest.mark.parametrize("case", CASES)
def test_decode_cases(case):
    nseq, Hq, Hkv, D, ps, lens = case
    say(f"decode nseq={nseq} Hq={Hq} Hkv={Hkv} D={D} ps={ps}")
    d = inputs.decode_inputs(nseq, Hq, Hkv, D, ps, 0, 0, "bf16", seed=nseq + Hq + D + ps, seq_lens=lens)
    scale = 1.0 / math.sqrt(D)
    check_bf16(f64(_run(d, scale)), _oracle(d, scale), str(case))


def test_many_short_sequences():
    d = inputs.decode_inputs(2000, 8, 2, 128, 16, 1, 40, "bf16", seed=31)
    scale = 0.1
    check_bf16(f64(_run(d, scale)), _oracle(d, scale), "2000 short sequences")


def test_permuted_pages_equal_identity_bit_exact():
    lens = [900, 17, 4000, 256]
    a = inputs.decode_inputs(4, 16, 4, 128, 16, 0, 0, "bf16", seed=32, seq_lens=lens, permute=False)
    b = inputs.decode_inputs(4, 16, 4, 128, 16, 0, 0, "bf16", seed=32, seq_lens=lens, permute=True)
    # same token values, scattered through the pool by the page table
    counts = [(n + 15) // 16 for n in lens]
    assert b["k_pool"].shape[0] == sum(counts)
    for name in ("k_pool", "v_pool"):
        src = a[name]
        dst = torch.empty_like(src)
        dst[b["page_table"].long()] = src[torch.arange(src.shape[0])]
        b[name] = dst
    b["q"] = a["q"]
    assert torch.equal(_run(a, 0.09), _run(b, 0.09))


def test_decode_equals_last_prefill_row():
    # one decode step over a cache of t tokens is row t-1 of a causal prefill
    # ("拆开 LLM（二）", KV-cache section: cached and full recomputation agree)
    S, Hq, Hkv, D, ps = 300, 8, 2, 128, 16
    q, k, v = inputs.prefill_inputs(1, Hq, Hkv, S, S, D, "bf16", 33)
    scale = 1.0 / math.sqrt(D)
    full = attn.fwd(*cuda(q, k, v), scale=scale, causal=True).cpu()
    for t in (1, 16, 17, 150, 300):
        n_pages = (t + ps - 1) // ps
        kp = torch.zeros(n_pages * ps, Hkv, D, dtype=torch.bfloat16)
        vp = torch.zeros_like(kp)
        kp[:t] = k[0, :, :t].transpose(0, 1)
        vp[:t] = v[0, :, :t].transpose(0, 1)
        kp = kp.view(n_pages, ps, Hkv, D).transpose(1, 2).contiguous()
        vp = vp.view(n_pages, ps, Hkv, D).transpose(1, 2).contiguous()
        d = dict(q=q[0, :, t - 1][None].contiguous(), k_pool=kp, v_pool=vp,
                 page_table=torch.arange(n_pages, dtype=torch.int32), seq_lens=torch.tensor([t], dtype=torch.int32))
        step = _run(d, scale)
        check_bf16(f64(step[0]), f64(full[0, :, t - 1]), f"t={t}")
        check_bf16(f64(step), _oracle(d, scale), f"t={t} vs oracle")


def test_paged_position_probe():
    # Q = 0: uniform weights; V slot of logical token t holds the bits of t
    lens, ps, D = [3, 16, 33, 1000], 16, 64
    d = inputs.decode_inputs(len(lens), 4, 2, D, ps, 0, 0, "bf16", seed=34, seq_lens=lens, nan_pad=True)
    d["q"] = torch.zeros_like(d["q"])
    first = 0
    for n in lens:
        c = (n + ps - 1) // ps
        for p in range(c):
            page = int(d["page_table"][first + p])
            for s in range(ps):
                t = p * ps + s
                if t < n:
                    bits = ((t >> torch.arange(D)) & 1).to(torch.bfloat16)
                    d["v_pool"][page, :, s] = bits
        first += c
    got = f64(_run(d, 1.0))
    for b, n in enumerate(lens):
        ts = np.arange(n)
        want = ((ts[:, None] >> np.arange(D)[None, :]) & 1).mean(0)
        rel = np.abs(got[b] - want[None]) / np.maximum(want[None], 1e-30)
        assert rel.max() <= 2 ** -8, (b, rel.max())


def test_repeated_calls_and_streams_agree():
    d = inputs.decode_inputs(8, 8, 2, 128, 16, 10, 900, "bf16", seed=35)
    first = _run(d, 0.1)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q, kp, vp, pt, sl = cuda(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"])
        o = attn.decode_paged(q, kp, vp, pt, sl, scale=0.1)
    s.synchronize()
    assert torch.equal(o.cpu(), first)
    # a larger call grows the workspace; a smaller one after it reuses it
    big = inputs.decode_inputs(200, 32, 8, 128, 16, 10, 300, "bf16", seed=36)
    check_bf16(f64(_run(big, 0.1)), _oracle(big, 0.1), "grown workspace")
    assert torch.equal(_run(d, 0.1), first)
    attn.release()
    assert torch.equal(_run(d, 0.1), first)


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.5])
def test_unusual_scales(scale):
    d = inputs.decode_inputs(5, 8, 2, 128, 16, 1, 700, "bf16", seed=37)
    check_bf16(f64(_run(d, scale)), _oracle(d, scale), f"scale {scale}")
    check_bf16(f64(_run_w(d, scale, 100)), _oracle_w(d, scale, 100), f"window 100, scale {scale}")
    # eight heads per K/V head (the MFMA kernel)
    d = inputs.decode_inputs(5, 16, 2, 128, 16, 1, 700, "bf16", seed=38)
    check_bf16(f64(_run(d, scale)), _oracle(d, scale), f"8 heads per K/V head, scale {scale}")
    check_bf16(f64(_run_w(d, scale, 100)), _oracle_w(d, scale, 100), f"8 heads, window 100, scale {scale}")


# ---- sliding-window decode ------------------------------------------------------

def test_window_decode_workload():
    # the 64-sequence workload with a 4096-token window (about half of the
    # sequences are longer than the window)
    w = inputs.WORKLOADS["paged_decode"]
    say("window decode workload paged_decode, window 4096")
    d = inputs.workload_inputs("paged_decode")
    scale = 1.0 / math.sqrt(w["D"])
    check_bf16(f64(_run_w(d, scale, 4096)), _oracle_w(d, scale, 4096), "paged_decode window 4096")


WINDOW_CASES = [
    # nseq, Hq, Hkv, D, page_size, lens, window
    (4, 8, 2, 128, 16, [15, 16, 17, 33], 1),
    (4, 8, 2, 128, 16, [15, 16, 17, 33], 16),
    (5, 32, 8, 128, 16, [500, 1, 64, 63, 1000], 17),
    (3, 4, 4, 64, 8, [1, 8, 9], 2),
    (3, 12, 12, 64, 64, [130, 64, 1], 100),
    (2, 16, 1, 128, 32, [700, 5], 256),     # MQA
    (2, 8, 2, 128, 256, [300, 1000], 333),
    (6, 8, 2, 128, 16, [3000, 2048, 4097, 17, 5000, 100], 2048),
    (64, 4, 2, 128, 16, list(range(1, 65)), 7),
    (4, 16, 2, 128, 16, [1, 31, 33, 2000], 40),
    (3, 32, 2, 64, 8, [700, 65, 5], 64),
    (2, 48, 1, 128, 32, [900, 40], 500),
]


@pytest.mark.parametrize("case", WINDOW_CASES)
def test_window_decode_cases(case):
    nseq, Hq, Hkv, D, ps, lens, window = case
    say(f"window decode {case}")
    d = inputs.decode_inputs(nseq, Hq, Hkv, D, ps, 0, 0, "bf16", seed=sum(lens) % 1000 + window, seq_lens=lens)
    scale = 1.0 / math.sqrt(D)
    check_bf16(f64(_run_w(d, scale, window)), _oracle_w(d, scale, window), str(case))


def test_window_zero_and_wide_windows_equal_plain_decode_bit_exact():
    d = inputs.decode_inputs(6, 8, 2, 128, 16, 1, 900, "bf16", seed=38)
    plain = _run(d, 0.1)
    assert torch.equal(_run_w(d, 0.1, 0), plain)
    # a window at least as long as every sequence covers the same blocks
    assert torch.equal(_run_w(d, 0.1, 900), plain)


def test_window_one_is_the_last_value_row_exactly():
    d = inputs.decode_inputs(5, 8, 2, 128, 16, 1, 300, "bf16", seed=39)
    got = _run_w(d, 0.1, 1)
    first = 0
    for b, n in enumerate(d["seq_lens"].tolist()):
        c = (n + 15) // 16
        page = int(d["page_table"][first + (n - 1) // 16])
        vrow = d["v_pool"][page, :, (n - 1) % 16]             # [Hkv, D]
        assert torch.equal(got[b], vrow.repeat_interleave(4, dim=0)), b
        first += c


def test_window_decode_equals_last_windowed_prefill_row():
    S, Hq, Hkv, D, ps, W = 300, 8, 2, 128, 16, 37
    q, k, v = inputs.prefill_inputs(1, Hq, Hkv, S, S, D, "bf16", 40)
    scale = 1.0 / math.sqrt(D)
    full = attn.fwd(*cuda(q, k, v), scale=scale, causal=True, window=W).cpu()
    for t in (1, 36, 37, 38, 150, 300):
        n_pages = (t + ps - 1) // ps
        kp = torch.zeros(n_pages * ps, Hkv, D, dtype=torch.bfloat16)
        vp = torch.zeros_like(kp)
        kp[:t] = k[0, :, :t].transpose(0, 1)
        vp[:t] = v[0, :, :t].transpose(0, 1)
        kp = kp.view(n_pages, ps, Hkv, D).transpose(1, 2).contiguous()
        vp = vp.view(n_pages, ps, Hkv, D).transpose(1, 2).contiguous()
        d = dict(q=q[0, :, t - 1][None].contiguous(), k_pool=kp, v_pool=vp,
                 page_table=torch.arange(n_pages, dtype=torch.int32), seq_lens=torch.tensor([t], dtype=torch.int32))
        step = _run_w(d, scale, W)
        check_bf16(f64(step[0]), f64(full[0, :, t - 1]), f"t={t}")
        check_bf16(f64(step), _oracle_w(d, scale, W), f"t={t} vs oracle")
