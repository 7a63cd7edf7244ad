"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

import sys

import numpy as np
import pytest
import torch

# Tolerances against the float64 oracle, on inputs rounded to the compute
# dtype before either side sees them.
BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3
F32_MAX_ABS = 1e-5

# Backward pass (bf16): per element |got - want| <= BWD_ELEM_REL * (|want| +
# rms(want)) and mean |got - want| <= BWD_MEAN_REL * rms(want). A CPU emulation
# of the kernels' roundings (P and dS to bf16 before the products, bf16 O in
# rowsum(dO * O), lse off by up to 2^-9, outputs to bf16) reaches 0.034 and
# 0.002 on causal, windowed and full shapes of 1024 rows with D = 64 and 128,
# and 0.089 and 0.0016 on the causal 4096-row GQA shape, where the first keys
# collect 4 heads x 4096 rounded terms whose sum nearly cancels.
BWD_ELEM_REL = 0.15
BWD_MEAN_REL = 5e-3
# Where every wanted gradient is exactly 0 (a key seen only by itself, scale 0)
# the kernels leave the float32 cancellation residue of dP - rowsum(dO * O),
# terms of size ~sqrt(D): about 1e-6 after the scale; allow 1e-4.
BWD_ZERO_ABS = 1e-4

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def say(*args):
    """Name the case on stdout before a GPU step, flushed."""
    print(*args, file=sys.stdout, flush=True)


def f64(t):
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()


def errors(got, want):
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    assert np.all(np.isfinite(err)), "non-finite output"
    return float(err.max()), float(err.mean())


def check_bf16(got, want, what=""):
    mx, mean = errors(got, want)
    assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max abs {mx:.3e}, mean abs {mean:.3e}"
    return mx, mean


def check_bf16_floor(got, want, what=""):
    """The bf16 bar above the output's own rounding floor.

    Where |O| reaches 2 and more (a sharp softmax under a large |scale|
    returns nearly one V row), rounding the exact result to bfloat16 alone
    moves it by up to half a bf16 spacing, 2^-7 on [2, 4) and 2^-6 on [4, 8),
    beyond the fixed 1e-2. So each element may differ from the float64 result
    by BF16_MAX_ABS plus |bf16(want) - want|, and the mean by BF16_MEAN_ABS
    plus the mean of that floor.
    """
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(np.asarray(got, dtype=np.float64) - want)
    assert np.all(np.isfinite(err)), f"{what}: non-finite output"
    floor = np.abs(torch.from_numpy(want).to(torch.bfloat16).double().numpy() - want)
    excess = float((err - floor).max())
    mean_excess = float(err.mean() - floor.mean())
    assert excess <= BF16_MAX_ABS and mean_excess <= BF16_MEAN_ABS, \
        f"{what}: max abs {err.max():.3e} ({excess:.3e} above the bf16 floor), mean abs {err.mean():.3e}"
    return excess, mean_excess


def check_f32(got, want, what=""):
    mx, _ = errors(got, want)
    assert mx <= F32_MAX_ABS, f"{what}: max abs {mx:.3e}"
    return mx


def cuda(*ts):
    return [t.cuda() for t in ts]


def check_grad(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    assert np.all(np.isfinite(err)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    if rms == 0.0:
        mx = float(err.max(initial=0.0))
        assert mx <= BWD_ZERO_ABS, f"{what}: expected zeros, max abs {mx:.3e}"
        return mx, 0.0
    worst = float(np.max(err / (np.abs(want) + rms)))
    mean = float(err.mean()) / rms
    assert worst <= BWD_ELEM_REL and mean <= BWD_MEAN_REL, \
        f"{what}: max err/(|want|+rms) {worst:.3e}, mean err/rms {mean:.3e}"
    return worst, mean
