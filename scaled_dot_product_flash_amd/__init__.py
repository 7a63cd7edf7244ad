"""Python binding of libattn.so (MI355X / gfx950 fused attention).

Argument marshalling only: each function checks that the tensors have the
dtype, device, layout and shapes the C ABI expects, passes their device
pointers and torch's current HIP stream, and raises ``RuntimeError`` with the
library's message when a call returns an error. Every arithmetic step runs in
the library's kernels; there is no fallback path. If ``libattn.so`` has not
been built the first call raises.

The C ABI is declared in ``include/attn.h``.
"""

import ctypes
import math
import os

__all__ = ["fwd", "fwd_f32", "bwd", "decode_paged", "strerror", "release", "library_path", "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

ATTN_OK = 0


def library_path():
    return os.path.join(_HERE, "libattn.so")


def load_library():
    """Load libattn.so once. torch is imported first so the library binds to
    the HIP runtime torch already uses (one runtime per process)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  (loads torch's libamdhip64 before ours)

    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m scaled_dot_product_flash_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("attn_fwd", "attn_fwd_f32"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
        fn.restype = i32
    for name in ("attn_fwd_lse", "attn_fwd_f32_lse"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
        fn.restype = i32
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp]
    lib.attn_decode_paged_noalloc.restype = i32
    lib.attn_decode_paged_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.attn_decode_paged_window.restype = i32
    lib.attn_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    lib.attn_fwd_paged.restype = i32
    lib.attn_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.attn_kv_append.restype = i32
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    lib.attn_bwd.restype = i32
    i64, pp = ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p)
    lib.attn_pages_create.argtypes = [i32, i32, pp]
    lib.attn_pages_create.restype = i32
    lib.attn_pages_destroy.argtypes = [vp]
    lib.attn_pages_destroy.restype = None
    lib.attn_pages_resize.argtypes = [vp, i64, i32]
    lib.attn_pages_resize.restype = i32
    lib.attn_pages_free_count.argtypes = [vp]
    lib.attn_pages_free_count.restype = i32
    lib.attn_pages_table.argtypes = [vp, vp, i32, vp, i64, vp, ctypes.POINTER(ctypes.c_int64)]
    lib.attn_pages_table.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_release.argtypes = []
    lib.attn_release.restype = None
    _LIB = lib
    return lib


def strerror(code):
    return load_library().attn_strerror(int(code)).decode()


def release():
    load_library().attn_release()


def _check(rc, what):
    if rc != ATTN_OK:
        raise RuntimeError(f"{what} failed ({rc}): {strerror(rc)}")


def _launch(t, entry, *args):
    """entry(*args, stream) with t's device current and torch's current stream
    on that device as the last argument (the device is switched only when it
    is not already current: the switch costs more than the launch)."""
    import torch

    dev = t.device.index
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if torch.cuda.current_device() != dev:
        with torch.cuda.device(dev):
            stream = raw(dev) if raw is not None else torch.cuda.current_stream(dev).cuda_stream
            return entry(*args, stream)
    stream = raw(dev) if raw is not None else torch.cuda.current_stream(dev).cuda_stream
    return entry(*args, stream)


def _need(t, name, dtype):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _prefill(entry, dtype, q, k, v, o, scale, causal, window, lse=False):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dtype)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    Hkv, Sk = k.shape[1], k.shape[2]
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", dtype)
    if o.shape != q.shape:
        raise ValueError("o must have the shape of q")
    if not (q.device == k.device == v.device == o.device):
        raise ValueError("all tensors must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if lse:
        out_lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
        rc = _launch(q, entry, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), out_lse.data_ptr(), B, Hq, Hkv,
                     Sq, Sk, D, float(scale), int(bool(causal)), int(window))
        _check(rc, entry.__name__)
        return o, out_lse
    rc = _launch(q, entry, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, Hq, Hkv, Sq, Sk, D,
                 float(scale), int(bool(causal)), int(window))
    _check(rc, entry.__name__)
    return o


def fwd_lse(q, k, v, o=None, scale=None, causal=False, window=0):
    """fwd plus the float32 log-sum-exp of each row, [B, Hq, Sq]: (o, lse)."""
    import torch

    return _prefill(load_library().attn_fwd_lse, torch.bfloat16, q, k, v, o, scale, causal, window, lse=True)


def fwd_f32_lse(q, k, v, o=None, scale=None, causal=False, window=0):
    """fwd_f32 plus the float32 log-sum-exp of each row, [B, Hq, Sq]: (o, lse)."""
    import torch

    return _prefill(load_library().attn_fwd_f32_lse, torch.float32, q, k, v, o, scale, causal, window, lse=True)


def fwd(q, k, v, o=None, scale=None, causal=False, window=0):
    """bf16 prefill attention: q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D] -> o [B,Hq,Sq,D]."""
    import torch

    return _prefill(load_library().attn_fwd, torch.bfloat16, q, k, v, o, scale, causal, window)


def fwd_f32(q, k, v, o=None, scale=None, causal=False, window=0):
    """float32 prefill attention with float32 arithmetic throughout."""
    import torch

    return _prefill(load_library().attn_fwd_f32, torch.float32, q, k, v, o, scale, causal, window)


def bwd(q, k, v, o, do, lse, scale=None, causal=False, window=0, dq=None, dk=None, dv=None):
    """Backward pass of fwd: (dq, dk, dv) for upstream gradient do.

    q, o, do [B,Hq,Sq,D] and k, v [B,Hkv,Sk,D] bfloat16; lse [B,Hq,Sq] float32
    as returned by fwd_lse with this o. dq, dk, dv are allocated when None.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(t, name, torch.bfloat16)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, D]")
    _need(lse, "lse", torch.float32)
    B, Hq, Sq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    if o.shape != q.shape or do.shape != q.shape:
        raise ValueError("o and do must have the shape of q")
    if tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be [B, Hq, Sq]")
    Hkv, Sk = k.shape[1], k.shape[2]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _need(t, name, torch.bfloat16)
        if t.shape != like.shape:
            raise ValueError(f"{name} must have the shape of {'q' if like is q else 'k'}")
    if len({t.device for t in (q, k, v, o, do, lse, dq, dk, dv)}) != 1:
        raise ValueError("all tensors must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = load_library()
    rc = _launch(q, lib.attn_bwd, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                 dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Sq, Sk, D, float(scale),
                 int(bool(causal)), int(window))
    _check(rc, "attn_bwd")
    return dq, dk, dv


def _decode_args(q, k_pool, v_pool, page_table, seq_lens, scale, o):
    import torch

    _need(q, "q", torch.bfloat16)
    _need(k_pool, "k_pool", torch.bfloat16)
    _need(v_pool, "v_pool", torch.bfloat16)
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or k_pool.dim() != 4 or k_pool.shape != v_pool.shape:
        raise ValueError("q must be [B,Hq,D] and the pools [num_pages,Hkv,page_size,D]")
    B, Hq, D = q.shape
    Hkv, ps = k_pool.shape[1], k_pool.shape[2]
    if k_pool.shape[3] != D or seq_lens.shape != (B,):
        raise ValueError("pool head dim or seq_lens length does not match q")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16)
    if o.shape != q.shape:
        raise ValueError("o must have the shape of q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return B, Hq, Hkv, D, ps, float(scale), o


def decode_paged(q, k_pool, v_pool, page_table, seq_lens, scale=None, o=None):
    """One decode step over a paged cache.

    q [B,Hq,D] bf16; k_pool / v_pool [num_pages,Hkv,page_size,D] bf16;
    page_table int32 (ragged, see include/attn.h); seq_lens [B] int32.
    """
    import torch

    lib = load_library()
    B, Hq, Hkv, D, ps, scale, o = _decode_args(q, k_pool, v_pool, page_table, seq_lens, scale, o)
    rc = _launch(q, lib.attn_decode_paged, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
                 seq_lens.data_ptr(), B, Hq, Hkv, D, ps, scale, o.data_ptr())
    _check(rc, "attn_decode_paged")
    return o


def decode_paged_noalloc(q, k_pool, v_pool, page_table, seq_lens, scale=None, o=None):
    """decode_paged through attn_decode_paged_noalloc: the library allocates
    nothing (its partials go to a fixed per-device scratch array; calls that
    overlap on one GPU race). ``o`` should be passed by callers that must not
    allocate either."""
    import torch

    lib = load_library()
    B, Hq, Hkv, D, ps, scale, o = _decode_args(q, k_pool, v_pool, page_table, seq_lens, scale, o)
    rc = _launch(q, lib.attn_decode_paged_noalloc, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                 page_table.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, ps, scale,
                 o.data_ptr())
    _check(rc, "attn_decode_paged_noalloc")
    return o


def decode_paged_window(q, k_pool, v_pool, page_table, seq_lens, window, scale=None, o=None):
    """decode_paged restricted to each sequence's `window` most recent tokens
    (window 0: no restriction)."""
    import torch

    lib = load_library()
    B, Hq, Hkv, D, ps, scale, o = _decode_args(q, k_pool, v_pool, page_table, seq_lens, scale, o)
    rc = _launch(q, lib.attn_decode_paged_window, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                 page_table.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, ps, scale,
                 int(window), o.data_ptr())
    _check(rc, "attn_decode_paged_window")
    return o


def kv_append(k_new, v_new, k_pool, v_pool, page_table, seq_lens):
    """Write each sequence's new token (k_new, v_new: [B,Hkv,D] bf16) into its
    page slot at position seq_lens[b] - 1 (see attn_kv_append)."""
    import torch

    lib = load_library()
    _need(k_new, "k_new", torch.bfloat16)
    _need(v_new, "v_new", torch.bfloat16)
    _need(k_pool, "k_pool", torch.bfloat16)
    _need(v_pool, "v_pool", torch.bfloat16)
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if k_new.dim() != 3 or k_new.shape != v_new.shape or k_pool.dim() != 4 or k_pool.shape != v_pool.shape:
        raise ValueError("k_new/v_new must be [B,Hkv,D] and the pools [num_pages,Hkv,page_size,D]")
    B, Hkv, D = k_new.shape
    if k_pool.shape[1] != Hkv or k_pool.shape[3] != D or seq_lens.shape != (B,):
        raise ValueError("k_new, the pools and seq_lens do not match")
    rc = _launch(k_new, lib.attn_kv_append, k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                 page_table.data_ptr(), seq_lens.data_ptr(), B, Hkv, D, k_pool.shape[2])
    _check(rc, "attn_kv_append")


class PagePool:
    """Host-side page allocator of a paged KV cache (attn_pages_* in
    include/attn.h): sequences keyed by int ids own ceil(len / page_size)
    pages of a global pool; ``table`` writes the ragged page table."""

    def __init__(self, num_pages, page_size):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.attn_pages_create(int(num_pages), int(page_size), ctypes.byref(h)), "attn_pages_create")
        self._h = h
        self._lib = lib
        self.num_pages = int(num_pages)
        self.page_size = int(page_size)

    def close(self):
        if self._h:
            self._lib.attn_pages_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def resize(self, seq_id, length):
        _check(self._lib.attn_pages_resize(self._h, int(seq_id), int(length)), "attn_pages_resize")

    def free_count(self):
        n = self._lib.attn_pages_free_count(self._h)
        _check(min(n, 0), "attn_pages_free_count")
        return n

    def table(self, seq_ids):
        """(page_table, seq_lens) as CPU int32 tensors for seq_ids, in order."""
        import torch

        ids = torch.tensor([int(x) for x in seq_ids], dtype=torch.int64)
        lens = torch.empty(len(ids), dtype=torch.int32)
        need = ctypes.c_int64(0)
        rc = self._lib.attn_pages_table(self._h, ids.data_ptr() if len(ids) else None, len(ids), None, 0,
                                        lens.data_ptr() if len(ids) else None, ctypes.byref(need))
        if rc not in (0, -2):  # SHAPE only reports the size needed
            _check(rc, "attn_pages_table")
        table = torch.empty(max(need.value, 1), dtype=torch.int32)
        _check(self._lib.attn_pages_table(self._h, ids.data_ptr() if len(ids) else None, len(ids),
                                          table.data_ptr(), need.value, lens.data_ptr() if len(ids) else None,
                                          ctypes.byref(need)), "attn_pages_table")
        return table[:need.value], lens


def fwd_paged(q, k_pool, v_pool, page_table, seq_lens, o=None, scale=None, causal=False, window=0, lse=False):
    """Prefill of q [B,Hq,Sq,D] (the newest Sq tokens of each sequence) against
    a paged cache (see attn_fwd_paged); returns o, or (o, lse) with lse=True."""
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16)
    _need(k_pool, "k_pool", torch.bfloat16)
    _need(v_pool, "v_pool", torch.bfloat16)
    _need(page_table, "page_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 4 or k_pool.dim() != 4 or k_pool.shape != v_pool.shape:
        raise ValueError("q must be [B,Hq,Sq,D] and the pools [num_pages,Hkv,page_size,D]")
    B, Hq, Sq, D = q.shape
    Hkv, ps = k_pool.shape[1], k_pool.shape[2]
    if k_pool.shape[3] != D or seq_lens.shape != (B,):
        raise ValueError("pool head dim or seq_lens length does not match q")
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", torch.bfloat16)
    if o.shape != q.shape:
        raise ValueError("o must have the shape of q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out_lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if lse else None
    rc = _launch(q, lib.attn_fwd_paged, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
                 seq_lens.data_ptr(), o.data_ptr(), out_lse.data_ptr() if lse else None, B, Hq, Hkv,
                 Sq, D, ps, float(scale), int(bool(causal)), int(window))
    _check(rc, "attn_fwd_paged")
    return (o, out_lse) if lse else o
