"""The library's host code under the address, undefined-behaviour and thread
sanitizers.

Every host source of libattn.so (the C ABI, the page pool and the launchers
in the kernel files) is compiled for the host only with ASan and UBSan and
linked against tests/native/hip_host_stub.cpp, a stand-in HIP runtime that
plays one 256-CU device, allocates "device" memory on the host heap and
checks every kernel launch against the hardware's grid limits instead of
running it. tests/native/abi_host_check.cpp then drives each entry point:
the documented error codes, a sweep over boundary values of every size and
mask argument, and the page pool under random resizes. Any sanitizer report
or launch-limit violation aborts the program. A second build with the thread
sanitizer runs tests/native/abi_threads_check.cpp: eight threads on four
streams calling every entry point at once, with workspaces that grow and one
shared page pool. CPU only.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
SOURCES = ["api.cpp", "pages.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode_paged.hip",
           "decode_noalloc.hip", "kv_append.hip", "backward.hip"]
# host-side sanitizer flags: each -fsanitize= sits right after -Xarch_host so
# the device side of a hipcc line never gets it
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
GXX_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _tool(name, fallback):
    return shutil.which(name) or (fallback if os.path.exists(fallback) else None)


# thread sanitizer (cannot be combined with the address sanitizer); its
# host objects come from clang, so the stand-in runtime, the driver and the
# link use clang too, for one sanitizer runtime throughout
HOST_TSAN = ["-Xarch_host", "-fsanitize=thread"]
CXX_TSAN = ["-fsanitize=thread"]


def _build(d, host_flags, cxx_name, cxx_fallback, cxx_flags, driver, extra_link=()):
    hipcc = _tool("hipcc", "/opt/rocm/bin/hipcc")
    gxx = _tool(cxx_name, cxx_fallback)
    if hipcc is None or gxx is None:
        pytest.skip(f"hipcc and {cxx_name} are needed")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs, procs = [], []
    for src in SOURCES:
        obj = str(d / (src + ".o"))
        cmd = [hipcc, "-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
               "-fPIC", "-fno-omit-frame-pointer", *host_flags, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p, src in zip(procs, SOURCES):
        out = p.communicate(timeout=600)[0]
        assert p.returncode == 0, f"{src}: {out[-3000:]}"
    # host-only objects reference their (absent) device images by name; give
    # the stand-in runtime empty ones to register
    nm = subprocess.run(["nm", "-u", *objs], capture_output=True, text=True, check=True).stdout
    fatbins = sorted(set(re.findall(r"\b(__hip_fatbin_\w+)", nm)))
    defs = d / "fatbins.c"
    defs.write_text("".join(f"char {n}[64];\n" for n in fatbins))
    exe = str(d / driver.replace(".cpp", ""))
    for src in ("hip_host_stub.cpp", driver):
        subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *cxx_flags, "-D__HIP_PLATFORM_AMD__",
                        "-I", "/opt/rocm/include", *inc, "-c", os.path.join(NATIVE, src), "-o",
                        str(d / (src + ".o"))], check=True, capture_output=True, text=True, timeout=300)
    subprocess.run([gxx, "-x", "c", "-c", str(defs), "-o", str(d / "fatbins.o")], check=True, timeout=60)
    subprocess.run([gxx, *cxx_flags, "-o", exe, *objs, str(d / "hip_host_stub.cpp.o"),
                    str(d / (driver + ".o")), str(d / "fatbins.o"), *extra_link],
                   check=True, capture_output=True, text=True, timeout=300)
    return exe


@pytest.fixture(scope="module")
def host_check(tmp_path_factory):
    return _build(tmp_path_factory.mktemp("host_san"), HOST_SAN, "g++", "/usr/bin/g++", GXX_SAN, "abi_host_check.cpp")


@pytest.fixture(scope="module")
def threads_check(tmp_path_factory):
    return _build(tmp_path_factory.mktemp("host_tsan"), HOST_TSAN, "/opt/rocm/llvm/bin/clang++",
                  "/opt/rocm/llvm/bin/clang++", CXX_TSAN, "abi_threads_check.cpp", ("-pthread",))


def test_host_code_under_sanitizers(host_check):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([host_check, "200000"], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-6000:])
    assert run.stdout.strip().endswith("host checks ok")
    launches = int(re.search(r"launches (\d+)", run.stdout).group(1))
    assert launches > 50000    # the sweep reached the launchers, not only validation


def test_dispatch_log(host_check):
    """ATTN_LOG=1: each launch decision of the dispatch examples is one
    "[attn]" line on stderr naming the kernel and its grid."""
    env = dict(os.environ, ATTN_LOG="1", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([host_check, "0"], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-3000:])
    lines = [ln for ln in run.stderr.splitlines() if ln.startswith("[attn] ")]
    text = "\n".join(lines)
    for want in ("prefill_pipe_kernel<8,128,pos,contiguous> B=4 Hq=32 Hkv=8 Sq=4096 Sk=4096 causal=1 window=0",
                 "prefill_pipe_kernel<4,64,pos,contiguous> B=8 Hq=12",
                 "prefill_pipe_kernel<4,128,neg,contiguous> B=1 Hq=16",
                 "prefill_pipe_kernel<8,128,pos,paged> B=8 Hq=32",
                 "prefill_f32_kernel<64> B=1 Hq=1",
                 "decode_split_kernel<128,4,pos> B=64 Hq=32 Hkv=8",
                 "decode_mfma_kernel<128,pos> B=8 Hq=64 Hkv=8",
                 "decode_merge_kernel<128>",
                 "bwd_dq_kernel<128> B=1 Hq=8 Hkv=2",
                 "bwd_dkdv_kernel<128>",
                 "kv_append_kernel B=4 Hkv=8 D=128 page_size=16"):
        assert want in text, (want, text[-3000:])
    assert all(" grid " in ln for ln in lines)
    # without the variable the library prints nothing
    env.pop("ATTN_LOG")
    quiet = subprocess.run([host_check, "0"], capture_output=True, text=True, timeout=600, env=env)
    assert quiet.returncode == 0 and "[attn]" not in quiet.stderr


def test_host_code_under_thread_sanitizer(threads_check):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    run = subprocess.run([threads_check, "200"], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-6000:])
    assert "ThreadSanitizer" not in run.stderr, run.stderr[-6000:]
    assert run.stdout.strip().startswith("thread checks ok")
    assert int(re.search(r"launches (\d+)", run.stdout).group(1)) > 8 * 200 * 9
