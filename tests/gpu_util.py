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


def check_f32(got, want, what=""):
    mx, _ = errors(got, want)
    assert mx <= F32_MAX_ABS, f"{what}: max abs {mx:.3e}"
    return mx


def cuda(*ts):
    return [t.cuda() for t in ts]
