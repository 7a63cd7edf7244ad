"""GPU parity of attn_fwd / attn_fwd_f32 against the float64 oracle.

Inputs come from the seeded generators and are rounded to the compute dtype
before either side sees them. Tolerances: bf16 max abs <= 1e-2 and mean abs
<= 1e-3; f32 max abs <= 1e-5. The full-size workloads are checked on whole
(batch, query head) slices, every query row, in the launch configuration the
benchmark times (same entry point, same sizes).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import check_bf16, check_f32, cuda, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run(q, k, v, causal, window, scale=None, f32=False):
    qd, kd, vd = cuda(q, k, v)
    fn = attn.fwd_f32 if f32 else attn.fwd
    o = fn(qd, kd, vd, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    return o.cpu()


def _full_check(B, Hq, Hkv, Sq, Sk, D, causal, window, dtype, seed, scale=None):
    say(f"prefill {dtype} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} causal={causal} window={window}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    got = _run(q, k, v, causal, window, scale, f32=(dtype == "f32"))
    want = oracle.attention(f64(q), f64(k), f64(v), scale, causal, window)
    if dtype == "f32":
        return check_f32(f64(got), want, "f32")
    return check_bf16(f64(got), want, "bf16")


def test_one_hip_runtime_in_process():
    attn.load_library()
    torch.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


# ---- the named workloads ---------------------------------------------------


def test_tiny_f32_workload():
    w = inputs.WORKLOADS["tiny_f32"]
    _full_check(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Sk"], w["D"], w["causal"], w["window"], "f32", w["seed"])


def test_gpt2_causal_workload():
    w = inputs.WORKLOADS["gpt2_causal"]
    _full_check(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Sk"], w["D"], w["causal"], w["window"], "bf16", w["seed"])


def _sampled_rows(Sq, rng, n=40):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, Sq // 2, Sq - 129, Sq - 128, Sq - 2, Sq - 1]
    rows = set(r for r in fixed if 0 <= r < Sq)
    rows.update(int(x) for x in rng.integers(0, Sq, n))
    return sorted(rows)


# Whole (batch, query head) slices of the two large workloads, every query
# row, in the launch configuration the benchmark times (same entry point, same
# sizes): for the 4k causal GQA workload one query head of each K/V head group
# spread over the batch, for the 16k sliding-window workload four heads over
# four K/V head groups. The bf16 bars apply to each slice as a whole.
FULL_SLICES = {
    "gqa_causal_4k": [(0, 0), (1, 7), (2, 10), (3, 13), (0, 16), (1, 23), (2, 26), (3, 29)],
    "swa_16k_w4k": [(0, 0), (0, 9), (0, 18), (0, 31)],
}


@pytest.mark.parametrize("name", ["gqa_causal_4k", "swa_16k_w4k"])
def test_full_size_workload_whole_heads(name):
    w = inputs.WORKLOADS[name]
    say(f"prefill workload {name}")
    q, k, v = inputs.workload_inputs(name)
    scale = 1.0 / math.sqrt(w["D"])
    got = _run(q, k, v, w["causal"], w["window"], scale)
    assert torch.isfinite(got.float()).all()
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))  # exact copies of the bf16 values
    for b, h in FULL_SLICES[name]:
        want = np.empty((w["Sq"], w["D"]))
        for r0 in range(0, w["Sq"], 2048):   # row chunks only bound the oracle's memory
            rows = np.arange(r0, min(w["Sq"], r0 + 2048))
            want[rows] = oracle.attention_rows(qn, kn, vn, b, h, rows, scale, w["causal"], w["window"])
        mx, mean = check_bf16(f64(got[b, h]), want, f"{name} b={b} h={h} (all {w['Sq']} rows)")
        say(f"  b={b} h={h}: max abs {mx:.3e}, mean abs {mean:.3e}")


# More causal items than workgroup slots, in (batch, kv head) groups too small
# to fill two dispatch rounds of an XCD: each XCD then takes its items heaviest
# query tile first across its groups. One shape per launch shape (D = 64 with
# four waves; D = 128 with four waves for at most 2048 keys, eight beyond). The output starts as
# NaN, so a work item that no workgroup took leaves non-finite rows.
@pytest.mark.parametrize("shape", [(16, 12, 12, 1024, 64), (12, 32, 8, 1024, 128), (2, 16, 16, 4096, 128)])
def test_weight_ordered_rounds_sampled_rows(shape):
    B, Hq, Hkv, S, D = shape
    say(f"prefill weight-ordered rounds B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, S, D, "bf16", 61)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = cuda(q, k, v)
    o = torch.full_like(qd, float("nan"))
    attn.fwd(qd, kd, vd, o=o, scale=scale, causal=True)
    torch.cuda.synchronize()
    got = o.cpu()
    assert torch.isfinite(got.float()).all()
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    rng = np.random.default_rng(1)
    for b, h in [(0, 0), (B - 1, Hq - 1), (B // 2, Hq // 2), (B - 1, 1)]:
        rows = _sampled_rows(S, rng)
        want = oracle.attention_rows(qn, kn, vn, b, h, rows, scale, True, 0)
        check_bf16(f64(got[b, h][rows]), want, f"b={b} h={h}")


# ---- ragged and small shapes ---------------------------------------------------

SHAPES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, window
    (1, 1, 1, 1, 1, 64, False, 0),
    (1, 1, 1, 1, 1, 128, True, 0),
    (2, 4, 4, 77, 77, 64, False, 0),
    (2, 4, 2, 77, 77, 128, True, 0),
    (1, 8, 1, 129, 129, 128, True, 0),      # MQA, one row past a 128-row tile
    (1, 8, 8, 200, 333, 64, False, 0),      # Sq != Sk, non-causal
    (1, 4, 2, 100, 300, 128, True, 0),      # bottom-right causal
    (1, 4, 1, 1, 513, 128, True, 0),        # one query row over a long cache
    (3, 6, 3, 257, 257, 64, True, 7),       # sliding window
    (1, 32, 8, 300, 300, 128, True, 1),     # window of one key
    (1, 2, 2, 130, 130, 128, True, 64),     # window of exactly one tile
    (1, 2, 1, 500, 700, 128, True, 100),    # window, Sq < Sk
    (1, 2, 2, 190, 190, 64, True, 5000),    # window wider than the sequence
    (1, 4, 2, 100, 150, 128, True, 8),      # first tile: some rows of a wave see no key
    (1, 2, 2, 60, 170, 64, True, 8),        # the same across a 128-key tile
    (2, 16, 4, 1000, 1000, 128, True, 0),
    (1, 4, 4, 1000, 1000, 64, True, 0),
    # fewer (batch, kv head) groups than XCDs: one query tile's heads per
    # chunk, dealt in snake order (the last rounds partly empty)
    (1, 8, 1, 2000, 2000, 128, True, 0),
    (1, 4, 2, 1300, 1300, 128, True, 0),
    (2, 8, 1, 1500, 1500, 64, True, 0),
    # D = 64 over long key ranges (many 64-key tiles per row block)
    (1, 2, 1, 300, 4400, 64, True, 0),
    (1, 2, 2, 4200, 4200, 64, True, 1000),
    # enough 256-row tiles for the eight-wave D = 128 kernel, ragged
    (4, 32, 8, 1000, 1000, 128, True, 0),
    (4, 32, 8, 777, 900, 128, True, 100),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shapes(shape, dtype):
    _full_check(*shape, dtype=dtype, seed=sum(shape[:6]))


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.5])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unusual_scales(scale, dtype):
    _full_check(1, 4, 2, 150, 150, 128, True, 0, dtype, seed=9, scale=scale)
    _full_check(1, 2, 2, 90, 90, 64, True, 11, dtype, seed=10, scale=scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sharp_softmax(dtype):
    """scale 2.5 at D = 128 gives logits up to |scale q.k| ~ 150, a nearly
    one-hot softmax and outputs as large as V itself.

    The fixed bars assume logits of the size 1/sqrt(D) produces (|scale q.k|
    below ~8). Rounding error grows with magnitude, so here the bound is
    derived from the arithmetic: float32 logits carry an absolute error
    proportional to their size, so the f32 bar is 1e-5 * L / 8 with L the
    largest |scale q.k|; for bf16, P and O are each rounded once with a
    relative error of at most 2^-9, bounding the error by
    2^-9 * (max|O| + max|V|) plus the float32 part.
    """
    scale = 2.5
    q, k, v = inputs.prefill_inputs(1, 4, 2, 150, 150, 128, dtype, 12)
    got = f64(_run(q, k, v, True, 0, scale, f32=(dtype == "f32")))
    qn, kn, vn = f64(q), f64(k), f64(v)
    want = oracle.attention(qn, kn, vn, scale, True, 0)
    L = max(float(np.abs(qn[0, h] @ kn[0, h // 2].T).max()) * abs(scale) for h in range(4))
    err = np.abs(got - want)
    f32_bar = 1e-5 * max(1.0, L / 8)
    if dtype == "f32":
        assert err.max() <= f32_bar, (err.max(), f32_bar)
    else:
        bar = 2.0 ** -9 * (np.abs(want).max() + np.abs(vn).max()) + f32_bar
        assert err.max() <= bar and err.mean() <= 1e-3, (err.max(), bar, err.mean())


# ---- invariants with exact answers -------------------------------------------------


def test_causal_row0_and_window1_are_exact():
    q, k, v = inputs.prefill_inputs(2, 8, 2, 300, 300, 128, "bf16", 21)
    o = _run(q, k, v, True, 0)
    rep = 4
    assert torch.equal(o[:, :, 0], v.repeat_interleave(rep, dim=1)[:, :, 0])
    o1 = _run(q, k, v, True, 1)
    assert torch.equal(o1, v.repeat_interleave(rep, dim=1))


@pytest.mark.parametrize("window", [0, 50])
def test_future_perturbation_is_bit_exact(window):
    # the causality test of the LLMs-from-scratch article (gsyq.cn, §5): change
    # every key/value after position i (and, with a window, before i-W+1);
    # rows up to i must not move at all
    q, k, v = inputs.prefill_inputs(1, 4, 2, 400, 400, 128, "bf16", 22)
    base = _run(q, k, v, True, window)
    for i in (0, 63, 64, 200, 399):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, i + 1:] += 10
        v2[:, :, i + 1:] += 10
        if window:
            lo = max(0, i - window + 1)
            k2[:, :, :lo] -= 10
            v2[:, :, :lo] -= 10
        pert = _run(q, k2, v2, True, window)
        assert torch.equal(pert[:, :, i], base[:, :, i]), i


def test_gqa_equals_mha_on_repeated_kv_bit_exact():
    q, k, v = inputs.prefill_inputs(2, 8, 2, 260, 260, 128, "bf16", 23)
    gqa = _run(q, k, v, True, 0)
    mha = _run(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous(), True, 0)
    assert torch.equal(gqa, mha)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37)])
def test_position_probe(causal, window):
    # Q = 0 makes the weights uniform over the visible keys; V[j, c] = bit c of
    # j (exact in bf16), so O[i, c] = (# visible j with bit c set) / (# visible)
    S, D = 300, 64
    q = torch.zeros(1, 2, S, D, dtype=torch.bfloat16)
    k = torch.randn(1, 1, S, D).to(torch.bfloat16)
    j = torch.arange(S)
    bits = ((j[:, None] >> torch.arange(D)[None, :]) & 1).to(torch.bfloat16)
    v = bits[None, None].contiguous()
    got = f64(_run(q, k, v, causal, window))[0, 0]
    want = np.zeros((S, D))
    for i in range(S):
        first = max(0, i + 1 - window) if window else 0
        last = i if causal else S - 1
        sel = bits[first:last + 1].double().numpy()
        want[i] = sel.sum(0) / (last - first + 1)
    # P is uniform, so only the final bf16 rounding of O separates the two
    assert np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30)) <= 2 ** -8


def test_o_is_not_written_outside_its_rows():
    q, k, v = inputs.prefill_inputs(1, 2, 2, 70, 70, 64, "bf16", 24)
    qd, kd, vd = cuda(q, k, v)
    big = torch.full((2 * 2 * 70 * 64 + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    o = big[:2 * 70 * 64].view(1, 2, 70, 64)
    attn.fwd(qd, kd, vd, o=o, causal=True)
    torch.cuda.synchronize()
    assert torch.all(big[2 * 70 * 64:] == 7.0)


# ---- log-sum-exp output ----------------------------------------------------------
# bf16 path: the row sum adds the bf16-rounded probabilities, each within 2^-9
# (relative) of the exact one, so |error of lse| <= -log(1 - 2^-9) < 2^-8;
# f32 path: float32 logits and sums, bar 1e-5 on the natural-log value.
LSE_BF16_BAR = 2.0 ** -8
LSE_F32_BAR = 1e-5

LSE_SHAPES = [
    (1, 1, 1, 1, 1, 64, False, 0),
    (2, 4, 2, 77, 77, 128, True, 0),
    (1, 8, 1, 129, 129, 128, True, 0),
    (1, 8, 8, 200, 333, 64, False, 0),
    (1, 4, 2, 100, 300, 128, True, 0),
    (3, 6, 3, 257, 257, 64, True, 7),
    (1, 2, 1, 500, 700, 128, True, 100),
    (2, 16, 4, 1000, 1000, 128, True, 0),
]


@pytest.mark.parametrize("shape", LSE_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lse_output(shape, dtype):
    B, Hq, Hkv, Sq, Sk, D, causal, window = shape
    say(f"lse {dtype} {shape}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed=sum(shape[:6]) + 5)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = cuda(q, k, v)
    fn = attn.fwd_f32_lse if dtype == "f32" else attn.fwd_lse
    o, lse = fn(qd, kd, vd, scale=scale, causal=causal, window=window)
    plain = (attn.fwd_f32 if dtype == "f32" else attn.fwd)(qd, kd, vd, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o, plain)            # the extra output changes nothing else
    want = oracle.attention_lse(f64(q), f64(k), f64(v), scale, causal, window)
    err = np.abs(f64(lse.cpu()) - want)
    bar = LSE_F32_BAR if dtype == "f32" else LSE_BF16_BAR
    assert err.max() <= bar, (err.max(), bar)


def test_lse_full_size_workload_whole_batch():
    # every row of every query head of one sequence of the 4k causal GQA
    # workload against the oracle's log-sum-exp
    w = inputs.WORKLOADS["gqa_causal_4k"]
    say("lse workload gqa_causal_4k, batch 1")
    q, k, v = inputs.workload_inputs("gqa_causal_4k")
    scale = 1.0 / math.sqrt(w["D"])
    o, lse = attn.fwd_lse(*cuda(q, k, v), scale=scale, causal=True)
    lse = lse.cpu()
    b = 1
    want = oracle.attention_lse(f64(q[b:b + 1]), f64(k[b:b + 1]), f64(v[b:b + 1]), scale, True, 0)
    err = np.abs(f64(lse[b:b + 1]) - want)
    assert err.max() <= LSE_BF16_BAR, err.max()


def test_lse_merges_two_key_halves():
    # the use of lse: attention over keys [0, n) equals the lse-weighted merge
    # of attention over [0, n/2) and [n/2, n) (non-causal halves)
    q, k, v = inputs.prefill_inputs(1, 4, 2, 64, 512, 128, "f32", 44)
    qd, kd, vd = cuda(q, k, v)
    o, _ = attn.fwd_f32_lse(qd, kd, vd)
    o1, l1 = attn.fwd_f32_lse(qd, kd[:, :, :256].contiguous(), vd[:, :, :256].contiguous())
    o2, l2 = attn.fwd_f32_lse(qd, kd[:, :, 256:].contiguous(), vd[:, :, 256:].contiguous())
    lm = torch.logaddexp(l1, l2)
    merged = o1 * torch.exp(l1 - lm)[..., None] + o2 * torch.exp(l2 - lm)[..., None]
    torch.cuda.synchronize()
    assert (merged - o).abs().max().item() <= 1e-5
