"""Host check of the work deal shared by the prefill and dQ kernels (deal.h).

tests/native/deal_check.cpp includes the header the kernels use, builds for
the host with hipcc, and enumerates every workgroup of the grid for 18 launch
shapes x paged/contiguous x causal/not x 1-3 workgroups per CU x 256/240 CUs:
each work item must be taken by exactly one workgroup (chunked snake deal,
one-round weight deal and several-round weight deal alike).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_item_dealt_exactly_once(tmp_path):
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = tmp_path / "deal_check"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc"), "-x", "hip",
                    os.path.join(ROOT, "tests", "native", "deal_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout[-2000:]
    assert run.stdout.strip().endswith("all shapes ok")
    assert "bal -1" in run.stdout and "bal 32" in run.stdout   # both weight deals exercised
