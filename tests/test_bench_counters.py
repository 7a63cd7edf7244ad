"""Host logic of bench.py's hardware-counter summary (no GPU): byte counters
scaled by the copy, MFMA utilisation over the SIMD cycles, decode GB/s."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _passes(copy_fetch_kib, copy_write_kib):
    n = 3
    pre = "void attn::prefill_pipe_kernel<8, false, false>(...)"
    split = "void attn::decode_split_kernel<128, 4, false>(...)"
    merge = "void attn::decode_merge_kernel<128>(...)"
    copy = "__amd_rocclr_copyBuffer"
    # prefill: 500 us at 2.0 GHz on 8 XCDs (GRBM_GUI_ACTIVE sums them), MFMA
    # busy half of 1024 SIMDs' cycles
    cycles = 2.0e9 * 500e-6
    fpass = {
        pre: [{"FETCH_SIZE": 100000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cycles * 1024, "SQ_INSTS_MFMA": 17e6,
               "GRBM_GUI_ACTIVE": 8 * cycles, "dur_ns": 500_000}] * n,
        split: [{"FETCH_SIZE": 600000.0, "dur_ns": 190_000}] * n,
        merge: [{"FETCH_SIZE": 2000.0, "dur_ns": 10_000}] * n,
        copy: [{"FETCH_SIZE": 3.0, "dur_ns": 1000}] + [{"FETCH_SIZE": copy_fetch_kib, "dur_ns": 50_000}] * n,
    }
    wpass = {
        pre: [{"WRITE_SIZE": 131072.0, "dur_ns": 500_000}] * n,
        split: [{"WRITE_SIZE": 4000.0, "dur_ns": 190_000}] * n,
        merge: [{"WRITE_SIZE": 500.0, "dur_ns": 10_000}] * n,
        copy: [{"WRITE_SIZE": copy_write_kib, "dur_ns": 50_000}] * n,
    }
    return fpass, wpass


def test_summary_arithmetic():
    b = _bench()
    fpass, wpass = _passes(131072.0, 262144.0)      # fetch reads half the copied bytes
    c = b.summarize_counters(fpass, wpass, 256)
    assert c["fetch_scale"] == pytest.approx(2.0) and c["write_scale"] == pytest.approx(1.0)
    p = c["prefill"]
    assert p["clock_ghz"] == pytest.approx(2.0)
    assert p["mfma_busy_frac"] == pytest.approx(0.5)
    assert p["mfma_busy_frac_at_2p4ghz"] == pytest.approx(0.5 * 2.0 / 2.4, rel=1e-3)
    assert p["hbm_bytes"] == 100000 * 1024 * 2 + 131072 * 1024
    d = c["decode"]
    want = (600000 + 2000) * 1024 * 2 + (4000 + 500) * 1024
    assert d["hbm_bytes"] == want
    assert d["hbm_gbps"] == pytest.approx(want / 200_000, rel=1e-4)


def test_summary_reports_missing_kernels():
    b = _bench()
    fpass, wpass = _passes(131072.0, 262144.0)
    del fpass[next(k for k in fpass if "decode_split" in k)]
    assert "error" in b.summarize_counters(fpass, wpass, 256)
    fpass, wpass = _passes(131072.0, 262144.0)
    for k in [k for k in fpass if "copyBuffer" in k]:
        del fpass[k]
    assert "error" in b.summarize_counters(fpass, wpass, 256)
