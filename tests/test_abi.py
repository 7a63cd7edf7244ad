"""The C ABI on the host: exported symbols and argument validation.

Validation runs before any HIP call, so every error path is exercised here
without a GPU. No call in this file reaches a kernel launch: each one either
fails validation or is an empty call.
"""

import ctypes
import os
import re
import subprocess

import pytest

import scaled_dot_product_flash_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, HEADS, HEADDIM, MASK, SCALE, PAGE, ALIGN, NOMEM, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10
FULL, SEQ, CAPTURE, SCRATCH = -11, -12, -13, -14


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def _codes():
    text = open(HEADER).read()
    return dict((n, int(v)) for n, v in re.findall(r"\b(ATTN_\w+)\s*=\s*(-?\d+)", text))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.library_path()):
        pytest.skip("libattn.so not built")
    return attn.load_library()


def test_header_declares_the_boundary():
    assert _declared() == ["attn_bwd", "attn_decode_paged", "attn_decode_paged_noalloc", "attn_decode_paged_window", "attn_fwd", "attn_fwd_f32",
                           "attn_fwd_f32_lse", "attn_fwd_lse", "attn_fwd_paged", "attn_kv_append", "attn_pages_create", "attn_pages_destroy", "attn_pages_free_count",
                           "attn_pages_resize", "attn_pages_table", "attn_release", "attn_strerror"]
    assert _codes() == {"ATTN_OK": OK, "ATTN_ERR_NULL": NULL, "ATTN_ERR_SHAPE": SHAPE, "ATTN_ERR_HEADS": HEADS,
                        "ATTN_ERR_HEADDIM": HEADDIM, "ATTN_ERR_MASK": MASK, "ATTN_ERR_SCALE": SCALE,
                        "ATTN_ERR_PAGE": PAGE, "ATTN_ERR_ALIGN": ALIGN, "ATTN_ERR_NOMEM": NOMEM, "ATTN_ERR_HIP": HIP,
                        "ATTN_ERR_FULL": FULL, "ATTN_ERR_SEQ": SEQ, "ATTN_ERR_CAPTURE": CAPTURE,
                        "ATTN_ERR_SCRATCH": SCRATCH}


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", attn.library_path()], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r"\bT (attn_\w+)$", out, flags=re.M)))
    assert exported == _declared()


def test_library_has_gfx950_code(lib):
    out = subprocess.run(["strings", attn.library_path()], capture_output=True, text=True).stdout
    assert "gfx950" in out


def test_strerror_covers_every_code(lib):
    msgs = set()
    for name, code in _codes().items():
        msg = attn.strerror(code)
        assert msg and "unknown" not in msg, name
        msgs.add(msg)
    assert len(msgs) == len(_codes())
    assert "unknown" in attn.strerror(12345)


A = 4096  # a 16-byte aligned, never dereferenced address
U = 4098  # a misaligned one


def _fwd(lib, q=A, k=A, v=A, o=A, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, D=64, scale=0.125, causal=1, window=0,
         f32=False):
    fn = lib.attn_fwd_f32 if f32 else lib.attn_fwd
    return fn(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, None)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL),
    (dict(B=-1), SHAPE), (dict(Sq=-3), SHAPE), (dict(Sk=0), SHAPE), (dict(Sq=9, Sk=8), SHAPE),
    (dict(Hq=0), HEADS), (dict(Hkv=0), HEADS), (dict(Hq=6, Hkv=4), HEADS),
    (dict(D=96), HEADDIM), (dict(D=256), HEADDIM), (dict(D=0), HEADDIM),
    (dict(causal=2), MASK), (dict(window=-1), MASK), (dict(causal=0, window=4), MASK),
    (dict(scale=float("nan")), SCALE), (dict(scale=float("inf")), SCALE), (dict(scale=-float("inf")), SCALE),
    (dict(q=U), ALIGN), (dict(k=U), ALIGN), (dict(v=U), ALIGN), (dict(o=U), ALIGN),
    (dict(B=1 << 30, Hq=1 << 20, Hkv=1, Sq=1 << 20, Sk=1 << 20), SHAPE),
])
def test_prefill_validation(lib, kwargs, code, f32):
    assert _fwd(lib, f32=f32, **kwargs) == code


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_longest_key_range_boundary(lib, D, f32):
    # the longest key range with Sk * D * 4 < 2^31 passes validation (the call
    # then stops at the HIP runtime, there being no GPU here); one key more is
    # a size error. tests/test_gpu_max_sizes.py runs the longest range.
    sk = (2 ** 31 - 1) // (D * 4)
    assert _fwd(lib, D=D, Sk=sk + 1, f32=f32) == SHAPE
    assert _fwd(lib, D=D, Sk=sk, f32=f32) == HIP


@pytest.mark.parametrize("f32", [False, True])
def test_prefill_empty_calls_are_no_ops(lib, f32):
    # nothing to compute: no pointer is needed and no HIP call is made
    assert _fwd(lib, q=None, k=None, v=None, o=None, B=0, f32=f32) == OK
    assert _fwd(lib, q=None, k=None, v=None, o=None, Sq=0, f32=f32) == OK
    assert _fwd(lib, q=None, k=None, v=None, o=None, Sq=0, causal=0, f32=f32) == OK


def _dec(lib, q=A, kp=A, vp=A, pt=A, sl=A, o=A, B=2, Hq=8, Hkv=2, D=128, ps=16, scale=0.1, window=None,
         noalloc=False):
    if noalloc:
        return lib.attn_decode_paged_noalloc(q, kp, vp, pt, sl, B, Hq, Hkv, D, ps, scale, o, None)
    if window is None:
        return lib.attn_decode_paged(q, kp, vp, pt, sl, B, Hq, Hkv, D, ps, scale, o, None)
    return lib.attn_decode_paged_window(q, kp, vp, pt, sl, B, Hq, Hkv, D, ps, scale, window, o, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), NULL), (dict(kp=None), NULL), (dict(vp=None), NULL), (dict(pt=None), NULL),
    (dict(sl=None), NULL), (dict(o=None), NULL),
    (dict(B=-1), SHAPE), (dict(B=70000), SHAPE), (dict(Hq=70000, Hkv=1), SHAPE),
    (dict(B=65535, Hq=512, Hkv=8), SHAPE),   # B * Hq > 2^24
    (dict(Hq=0), HEADS), (dict(Hkv=0), HEADS), (dict(Hq=8, Hkv=3), HEADS),
    (dict(D=32), HEADDIM),
    (dict(ps=0), PAGE), (dict(ps=4), PAGE), (dict(ps=12), PAGE), (dict(ps=512), PAGE), (dict(ps=-16), PAGE),
    (dict(scale=float("nan")), SCALE),
    (dict(q=U), ALIGN), (dict(kp=U), ALIGN), (dict(vp=U), ALIGN), (dict(o=U), ALIGN), (dict(pt=A + 2), ALIGN),
    (dict(sl=A + 1), ALIGN),
])
def test_decode_validation(lib, kwargs, code):
    assert _dec(lib, **kwargs) == code
    # the windowed and the allocation-free entry points validate the same
    # arguments the same way
    assert _dec(lib, window=5, **kwargs) == code
    assert _dec(lib, noalloc=True, **kwargs) == code


@pytest.mark.parametrize("B,Hq,Hkv,D", [(32264, 1, 1, 128), (1000, 33, 1, 128), (64, 1024, 8, 128),
                                        (16384, 4, 4, 64)])
def test_decode_noalloc_scratch_limit(lib, B, Hq, Hkv, D):
    # B * Hq * (D + 2) * 4 bytes above the 16 MiB scratch: refused before any
    # HIP call; one fewer (sequence, head) unit than the limit passes that check
    assert B * Hq * (D + 2) * 4 > 16 << 20
    assert _dec(lib, B=B, Hq=Hq, Hkv=Hkv, D=D, noalloc=True) == SCRATCH
    assert _dec(lib, B=B, Hq=Hq, Hkv=Hkv, D=D, noalloc=True, q=None) == NULL  # validated first


def test_decode_noalloc_empty_batch_is_a_no_op(lib):
    assert _dec(lib, q=None, kp=None, vp=None, pt=None, sl=None, o=None, B=0, noalloc=True) == OK


@pytest.mark.parametrize("window", [-1, -100])
def test_decode_window_validation(lib, window):
    assert _dec(lib, window=window) == MASK
    assert _dec(lib, window=window, B=0) == MASK


def test_decode_empty_batch_is_a_no_op(lib):
    assert _dec(lib, q=None, kp=None, vp=None, pt=None, sl=None, o=None, B=0) == OK
    assert _dec(lib, q=None, kp=None, vp=None, pt=None, sl=None, o=None, B=0, window=3) == OK


def test_release_without_work_is_a_no_op(lib):
    lib.attn_release()
    lib.attn_release()


def test_binding_rejects_cpu_tensors(lib):
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.fwd(q, q, q)
    with pytest.raises(ValueError):
        attn.decode_paged(q[0], q, q, torch.zeros(1, dtype=torch.int32), torch.ones(1, dtype=torch.int32))


def test_ctypes_signature_matches_header(lib):
    assert lib.attn_fwd.restype is ctypes.c_int
    assert len(lib.attn_fwd.argtypes) == 14
    assert len(lib.attn_decode_paged.argtypes) == 13
    assert len(lib.attn_decode_paged_window.argtypes) == 14
    assert len(lib.attn_fwd_lse.argtypes) == len(lib.attn_fwd_f32_lse.argtypes) == 15
    assert len(lib.attn_bwd.argtypes) == 19


def _app(lib, kn=A, vn=A, kp=A, vp=A, pt=A, sl=A, B=2, Hkv=2, D=128, ps=16):
    return lib.attn_kv_append(kn, vn, kp, vp, pt, sl, B, Hkv, D, ps, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(kn=None), NULL), (dict(vn=None), NULL), (dict(kp=None), NULL), (dict(vp=None), NULL),
    (dict(pt=None), NULL), (dict(sl=None), NULL),
    (dict(B=-1), SHAPE), (dict(Hkv=0), HEADS), (dict(D=96), HEADDIM),
    (dict(ps=4), PAGE), (dict(ps=24), PAGE), (dict(ps=512), PAGE),
    (dict(kn=U), ALIGN), (dict(vn=U), ALIGN), (dict(kp=U), ALIGN), (dict(vp=U), ALIGN), (dict(pt=A + 2), ALIGN),
    (dict(sl=A + 1), ALIGN),
])
def test_kv_append_validation(lib, kwargs, code):
    assert _app(lib, **kwargs) == code


def test_kv_append_empty_batch_is_a_no_op(lib):
    assert _app(lib, kn=None, vn=None, kp=None, vp=None, pt=None, sl=None, B=0) == OK


def test_page_pool_argument_errors(lib):
    h = ctypes.c_void_p()
    assert lib.attn_pages_create(0, 16, ctypes.byref(h)) == SHAPE
    assert lib.attn_pages_create(4, 12, ctypes.byref(h)) == PAGE
    assert lib.attn_pages_create(4, 16, None) == NULL
    assert lib.attn_pages_resize(None, 1, 3) == NULL
    assert lib.attn_pages_free_count(None) == NULL
    n = ctypes.c_int64(0)
    assert lib.attn_pages_table(None, None, 0, None, 0, None, ctypes.byref(n)) == NULL
    lib.attn_pages_destroy(None)
    assert lib.attn_pages_create(4, 16, ctypes.byref(h)) == OK
    try:
        assert lib.attn_pages_resize(h, 1, -1) == SHAPE
        assert lib.attn_pages_resize(h, 1, 4 * 16 + 1) == FULL
        assert lib.attn_pages_free_count(h) == 4
        ids = (ctypes.c_int64 * 1)(99)
        lens = (ctypes.c_int32 * 1)()
        assert lib.attn_pages_table(h, ids, 1, None, 0, lens, ctypes.byref(n)) == SEQ
        assert lib.attn_pages_resize(h, 99, 20) == OK
        assert lib.attn_pages_table(h, ids, 1, None, 0, lens, ctypes.byref(n)) == SHAPE and n.value == 2
        assert lib.attn_pages_table(h, ids, -1, None, 0, lens, ctypes.byref(n)) == SHAPE
    finally:
        lib.attn_pages_destroy(h)


def _fwd_lse(lib, lse=A, f32=False, **kw):
    args = dict(q=A, k=A, v=A, o=A, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, D=64, scale=0.125, causal=1, window=0)
    args.update(kw)
    fn = lib.attn_fwd_f32_lse if f32 else lib.attn_fwd_lse
    return fn(args["q"], args["k"], args["v"], args["o"], lse, args["B"], args["Hq"], args["Hkv"], args["Sq"],
              args["Sk"], args["D"], args["scale"], args["causal"], args["window"], None)


@pytest.mark.parametrize("f32", [False, True])
def test_fwd_lse_validation(lib, f32):
    assert _fwd_lse(lib, lse=None, f32=f32) == NULL
    assert _fwd_lse(lib, lse=A + 2, f32=f32) == ALIGN
    # the arguments shared with attn_fwd are checked the same way, first
    assert _fwd_lse(lib, f32=f32, D=96) == HEADDIM
    assert _fwd_lse(lib, f32=f32, causal=0, window=3) == MASK
    assert _fwd_lse(lib, f32=f32, q=None) == NULL
    # empty calls need no pointer at all
    assert _fwd_lse(lib, lse=None, f32=f32, q=None, k=None, v=None, o=None, B=0) == OK
    assert _fwd_lse(lib, lse=None, f32=f32, q=None, k=None, v=None, o=None, Sq=0) == OK


def _fwdp(lib, q=A, kp=A, vp=A, pt=A, sl=A, o=A, lse=None, B=2, Hq=8, Hkv=2, Sq=16, D=128, ps=16, scale=0.1,
          causal=1, window=0):
    return lib.attn_fwd_paged(q, kp, vp, pt, sl, o, lse, B, Hq, Hkv, Sq, D, ps, scale, causal, window, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), NULL), (dict(kp=None), NULL), (dict(vp=None), NULL), (dict(pt=None), NULL),
    (dict(sl=None), NULL), (dict(o=None), NULL),
    (dict(B=-1), SHAPE), (dict(Sq=-1), SHAPE),
    (dict(Hq=0), HEADS), (dict(Hq=8, Hkv=3), HEADS), (dict(D=32), HEADDIM), (dict(D=96), HEADDIM),
    (dict(ps=4), PAGE), (dict(ps=48), PAGE), (dict(causal=2), MASK), (dict(causal=0, window=3), MASK),
    (dict(window=-2), MASK), (dict(scale=float("nan")), SCALE),
    (dict(q=U), ALIGN), (dict(kp=U), ALIGN), (dict(o=U), ALIGN), (dict(pt=A + 2), ALIGN), (dict(lse=A + 2), ALIGN),
])
def test_fwd_paged_validation(lib, kwargs, code):
    assert _fwdp(lib, **kwargs) == code


def test_fwd_paged_empty_calls(lib):
    assert _fwdp(lib, q=None, kp=None, vp=None, pt=None, sl=None, o=None, B=0) == OK
    assert _fwdp(lib, q=None, kp=None, vp=None, pt=None, sl=None, o=None, Sq=0) == OK


def _bwd(lib, q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, D=128, scale=0.1,
         causal=1, window=0):
    return lib.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, scale, causal, window, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL), (dict(do=None), NULL),
    (dict(lse=None), NULL), (dict(dq=None), NULL), (dict(dk=None), NULL), (dict(dv=None), NULL),
    (dict(B=-1), SHAPE), (dict(Sq=-1), SHAPE), (dict(Sk=-1), SHAPE), (dict(Sk=0), SHAPE),
    (dict(Sq=9, Sk=8), SHAPE), (dict(Sk=1 << 23), SHAPE), (dict(Sq=1 << 23, Sk=1 << 23, causal=0), SHAPE),
    (dict(Hq=0), HEADS), (dict(Hkv=3), HEADS), (dict(D=96), HEADDIM),
    (dict(causal=2), MASK), (dict(causal=0, window=4), MASK), (dict(window=-1), MASK),
    (dict(scale=float("inf")), SCALE),
    (dict(q=U), ALIGN), (dict(k=U), ALIGN), (dict(v=U), ALIGN), (dict(o=U), ALIGN), (dict(do=U), ALIGN),
    (dict(lse=A + 2), ALIGN), (dict(dq=U), ALIGN), (dict(dk=U), ALIGN), (dict(dv=U), ALIGN),
])
def test_bwd_validation(lib, kwargs, code):
    assert _bwd(lib, **kwargs) == code


def test_bwd_empty_calls(lib):
    none = dict(q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None)
    assert _bwd(lib, B=0, **none) == OK
    assert _bwd(lib, Sq=0, Sk=0, causal=0, **none) == OK
    # Sq = 0 with keys still owes zero dk, dv: those two pointers are required
    assert _bwd(lib, Sq=0, **none) == NULL
    assert _bwd(lib, Sq=0, **dict(none, dk=A)) == NULL
    assert _bwd(lib, Sq=0, **dict(none, dk=A, dv=U)) == ALIGN
