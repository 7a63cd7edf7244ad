"""attn_decode_paged_noalloc through the C ABI against attn_decode_paged.

The allocation-free entry point runs the decode kernels with their partials
in a fixed per-device scratch array instead of the library's workspace. Two
calls in a row on the same device (the second with a smaller input, so it
reads partials the first left behind only if it were wrong) must each match
the plain entry point's output within the bf16 bars, and the float64 oracle.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import check_bf16, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]

NAMES = ("q", "k_pool", "v_pool", "page_table", "seq_lens")


def _call(fn, d, o, Hkv, ps, scale):
    q, kp, vp, pt, sl = d
    B, Hq, D = q.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(q.data_ptr(), kp.data_ptr(), vp.data_ptr(), pt.data_ptr(), sl.data_ptr(), B, Hq, Hkv, D, ps,
              scale, o.data_ptr(), stream)


@pytest.mark.parametrize("second", [(8, 16, 4, 64, 16, 1, 700), (3, 8, 8, 128, 32, 1, 90)])
def test_noalloc_decode_matches_plain_decode_twice(second):
    lib = attn.load_library()
    cases = [
        # the paged decode workload (64 sequences, lengths 512-8192, 32/8 heads,
        # D 128, pages of 16), then a smaller input
        ("paged_decode", inputs.workload_inputs("paged_decode"), 8, 16),
        ("smaller " + str(second), inputs.decode_inputs(*second, "bf16", seed=91), second[2], second[4]),
    ]
    for what, host, Hkv, ps in cases:
        say(f"decode_paged_noalloc: {what}")
        d = [host[n].cuda() for n in NAMES]
        scale = 1.0 / math.sqrt(d[0].shape[2])
        o_plain = torch.full_like(d[0], float("nan"))
        o_free = torch.full_like(d[0], float("nan"))
        assert _call(lib.attn_decode_paged, d, o_plain, Hkv, ps, scale) == 0
        rc = _call(lib.attn_decode_paged_noalloc, d, o_free, Hkv, ps, scale)
        assert rc == 0, attn.strerror(rc)
        torch.cuda.synchronize()
        assert torch.isfinite(o_free.float()).all()
        check_bf16(f64(o_free.cpu()), f64(o_plain.cpu()), f"{what}: noalloc vs plain")
        want = oracle.decode_paged(host["q"].double().numpy(), host["k_pool"].float().numpy(),
                                   host["v_pool"].float().numpy(), host["page_table"].numpy(),
                                   host["seq_lens"].numpy(), ps, scale)
        check_bf16(f64(o_free.cpu()), want, f"{what}: noalloc vs oracle")
