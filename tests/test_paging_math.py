"""Host replay of the paged-cache addressing (tests/native/paging_check.cpp).

The decode kernels (vector and MFMA), the paged prefill and the KV append
take their page-table and pool offsets from csrc/paging.h; the check program
includes that header, runs the kernels' loops over splits, blocks, tiles, DMA
slots and lanes on the host for 300 random ragged caches, and asserts that
every table read stays in the sequence's own entries, every element read in
the pool, every row is its token's row (compared with the layout written out
independently), and that the decode loops visit each visible token once.
CPU only.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_paged_addressing_replay(tmp_path):
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = tmp_path / "paging_check"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc"), "-x", "hip",
                    os.path.join(ROOT, "tests", "native", "paging_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout[-3000:]
    assert run.stdout.strip().endswith("random caches ok")
