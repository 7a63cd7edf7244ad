"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: it only draws random tensors,
rounds them to the compute dtype and lays out the paged KV cache. Both the GPU
path and the float64 oracle consume exactly the tensors it returns.

Recipe: a CPU ``torch.Generator`` seeded per workload draws float32 N(0, 1)
values (the pages' workloads are random tensors too), which are rounded to
bfloat16 with round-to-nearest-even when the workload is bf16. Draw order is
Q, K, V for prefill (then dO for the backward pass); lengths, page permutation, Q, K pool, V pool for decode.
"""

import math

import torch

# Named workloads. Seeds are 123 + index.
WORKLOADS = {
    "tiny_f32": dict(kind="prefill", B=1, Hq=1, Hkv=1, Sq=128, Sk=128, D=64,
                     dtype="f32", causal=False, window=0, seed=123),
    "gpt2_causal": dict(kind="prefill", B=8, Hq=12, Hkv=12, Sq=1024, Sk=1024, D=64,
                        dtype="bf16", causal=True, window=0, seed=124),
    "gqa_causal_4k": dict(kind="prefill", B=4, Hq=32, Hkv=8, Sq=4096, Sk=4096, D=128,
                          dtype="bf16", causal=True, window=0, seed=125),
    "paged_decode": dict(kind="decode", nseq=64, Hq=32, Hkv=8, D=128, page_size=16,
                         len_lo=512, len_hi=8192, dtype="bf16", seed=126),
    "swa_16k_w4k": dict(kind="prefill", B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384, D=128,
                        dtype="bf16", causal=True, window=4096, seed=127),
    # chunked prefill: 512 new tokens per sequence against paged caches of
    # 2048..6144 tokens (the new ones included)
    # backward pass on the causal GQA prefill shape; dO is the fourth draw
    "gqa_causal_4k_bwd": dict(kind="backward", B=4, Hq=32, Hkv=8, Sq=4096, Sk=4096, D=128,
                              dtype="bf16", causal=True, window=0, seed=129),
    "chunked_prefill_paged": dict(kind="paged_prefill", nseq=8, Sq=512, Hq=32, Hkv=8, D=128, page_size=16,
                                  len_lo=2048, len_hi=6144, dtype="bf16", seed=128),
}


def _torch_dtype(dtype):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def prefill_inputs(B, Hq, Hkv, Sq, Sk, D, dtype="bf16", seed=0):
    """q [B,Hq,Sq,D], k and v [B,Hkv,Sk,D] on the CPU, i.i.d. N(0,1) then rounded."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    td = _torch_dtype(dtype)
    q = torch.randn((B, Hq, Sq, D), generator=g, dtype=torch.float32).to(td)
    k = torch.randn((B, Hkv, Sk, D), generator=g, dtype=torch.float32).to(td)
    v = torch.randn((B, Hkv, Sk, D), generator=g, dtype=torch.float32).to(td)
    return q, k, v


def backward_inputs(B, Hq, Hkv, Sq, Sk, D, seed=0):
    """q, k, v as prefill_inputs (bf16) plus an upstream gradient do
    [B,Hq,Sq,D], i.i.d. N(0,1) drawn after them from the same generator."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((B, Hq, Sq, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Sk, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Sk, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    do = torch.randn((B, Hq, Sq, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do


def page_counts(seq_lens, page_size):
    return [(int(n) + page_size - 1) // page_size for n in seq_lens]


def decode_inputs(nseq, Hq, Hkv, D, page_size, len_lo, len_hi, dtype="bf16", seed=0,
                  seq_lens=None, permute=True, nan_pad=True):
    """A paged KV cache plus one query token per sequence, all on the CPU.

    Lengths are uniform integers in [len_lo, len_hi] unless ``seq_lens`` is
    given. The pool holds exactly sum(ceil(len / page_size)) pages; the ragged
    page table lists each sequence's physical pages in logical order and is a
    seeded random permutation of the pool (identity if ``permute`` is False).
    Slots past a sequence's length are filled with NaN when ``nan_pad`` is
    set, so any read of them shows up in the output.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    td = _torch_dtype(dtype)
    if seq_lens is None:
        seq_lens = torch.randint(len_lo, len_hi + 1, (nseq,), generator=g, dtype=torch.int64)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    counts = page_counts(seq_lens.tolist(), page_size)
    num_pages = sum(counts)
    if permute:
        table = torch.randperm(num_pages, generator=g)
    else:
        table = torch.arange(num_pages)
    q = torch.randn((nseq, Hq, D), generator=g, dtype=torch.float32).to(td)
    k_pool = torch.randn((num_pages, Hkv, page_size, D), generator=g, dtype=torch.float32).to(td)
    v_pool = torch.randn((num_pages, Hkv, page_size, D), generator=g, dtype=torch.float32).to(td)
    if nan_pad:
        first = 0
        for n, c in zip(seq_lens.tolist(), counts):
            tail = c * page_size - n
            if tail:
                last = int(table[first + c - 1])
                k_pool[last, :, page_size - tail:, :] = float("nan")
                v_pool[last, :, page_size - tail:, :] = float("nan")
            first += c
    return dict(q=q, k_pool=k_pool, v_pool=v_pool,
                page_table=table.to(torch.int32), seq_lens=seq_lens.to(torch.int32))


def paged_prefill_inputs(nseq, Sq, Hq, Hkv, D, page_size, len_lo, len_hi, dtype="bf16", seed=0):
    """A paged cache as in decode_inputs (drawn first, same seed) plus q
    [nseq, Hq, Sq, D] for the Sq newest tokens of each sequence."""
    d = decode_inputs(nseq, Hq, Hkv, D, page_size, len_lo, len_hi, dtype, seed)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    d["q"] = torch.randn((nseq, Hq, Sq, D), generator=g, dtype=torch.float32).to(_torch_dtype(dtype))
    return d


def workload_inputs(name):
    w = WORKLOADS[name]
    if w["kind"] == "paged_prefill":
        return paged_prefill_inputs(w["nseq"], w["Sq"], w["Hq"], w["Hkv"], w["D"], w["page_size"],
                                    w["len_lo"], w["len_hi"], w["dtype"], w["seed"])
    if w["kind"] == "backward":
        return backward_inputs(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Sk"], w["D"], w["seed"])
    if w["kind"] == "prefill":
        return prefill_inputs(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Sk"], w["D"],
                              w["dtype"], w["seed"])
    return decode_inputs(w["nseq"], w["Hq"], w["Hkv"], w["D"], w["page_size"],
                         w["len_lo"], w["len_hi"], w["dtype"], w["seed"])


def default_scale(D):
    return 1.0 / math.sqrt(D)
