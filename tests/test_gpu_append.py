"""GPU checks of attn_kv_append and of the page pool driving a decode loop.

The append is a copy, so its parity bar is bit-exact: the pools after the
kernel equal the float64 oracle's (every bf16 value is exact in float64),
NaN padding included.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import check_bf16, cuda, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _bits_equal(got, want):
    """Bitwise equality of bf16 tensors, except that a NaN of the oracle (whose
    float64 -> bf16 conversion picks its own NaN encoding) only asks for a NaN."""
    nan = torch.isnan(want)
    if not torch.equal(torch.isnan(got), nan):
        return False
    return torch.equal(got.view(torch.int16)[~nan], want.view(torch.int16)[~nan])


@pytest.mark.parametrize("case", [
    # nseq, Hkv, D, page_size, len_lo, len_hi
    (64, 8, 128, 16, 512, 8192),
    (5, 2, 64, 8, 1, 40),
    (3, 1, 128, 256, 1, 600),
    (300, 4, 128, 32, 1, 200),
])
def test_append_matches_oracle_bit_exact(case):
    nseq, Hkv, D, ps, lo, hi = case
    say(f"kv_append {case}")
    d = inputs.decode_inputs(nseq, 2 * Hkv, Hkv, D, ps, lo, hi, "bf16", seed=41 + nseq)
    g = torch.Generator().manual_seed(7)
    kn = torch.randn((nseq, Hkv, D), generator=g).to(torch.bfloat16)
    vn = torch.randn((nseq, Hkv, D), generator=g).to(torch.bfloat16)
    kp, vp, pt, sl, kn_d, vn_d = cuda(d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"], kn, vn)
    attn.kv_append(kn_d, vn_d, kp, vp, pt, sl)
    torch.cuda.synchronize()
    wk, wv = oracle.kv_append(kn.float().numpy(), vn.float().numpy(), d["k_pool"].float().numpy(),
                              d["v_pool"].float().numpy(), d["page_table"].numpy(), d["seq_lens"].numpy(), ps)
    assert _bits_equal(kp.cpu(), torch.from_numpy(wk).to(torch.bfloat16))
    assert _bits_equal(vp.cpu(), torch.from_numpy(wv).to(torch.bfloat16))


def test_pool_append_decode_loop_equals_causal_prefill():
    # three sequences grow token by token: the pool hands out pages, the
    # kernel appends each new k/v, the decode of each step must equal the
    # matching row of causal attention over the whole sequence (oracle)
    Hq, Hkv, D, ps = 8, 2, 128, 16
    lens = [70, 33, 1]
    steps = max(lens)
    q, k, v = inputs.prefill_inputs(len(lens), Hq, Hkv, steps, steps, D, "bf16", 42)
    scale = 1.0 / math.sqrt(D)
    full = oracle.attention(f64(q), f64(k), f64(v), scale, causal=True)   # float64 [B, Hq, S, D]
    pool = attn.PagePool(32, ps)
    k_pool = torch.full((32, Hkv, ps, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.full_like(k_pool, float("nan"))
    qd, kd, vd = cuda(q, k, v)
    for t in range(1, steps + 1):
        live = [b for b, n in enumerate(lens) if n >= t]
        for b in live:
            pool.resize(b, t)
        table, sl = pool.table(live)
        table_d, sl_d = cuda(table, sl)
        idx = torch.tensor(live, device="cuda")
        attn.kv_append(kd[idx, :, t - 1].contiguous(), vd[idx, :, t - 1].contiguous(), k_pool, v_pool,
                       table_d, sl_d)
        o = attn.decode_paged(qd[idx, :, t - 1].contiguous(), k_pool, v_pool, table_d, sl_d, scale=scale)
        torch.cuda.synchronize()
        check_bf16(f64(o.cpu()), full[live, :, t - 1], f"step {t}")
    # sequences that ended release their pages
    for b in range(len(lens)):
        pool.resize(b, 0)
    assert pool.free_count() == 32
    pool.close()


def test_append_leaves_other_slots_untouched():
    d = inputs.decode_inputs(6, 8, 2, 128, 16, 1, 100, "bf16", seed=43, nan_pad=True)
    kp, vp, pt, sl = cuda(d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"])
    before_k, before_v = kp.clone(), vp.clone()
    kn = torch.ones((6, 2, 128), dtype=torch.bfloat16, device="cuda")
    attn.kv_append(kn, kn, kp, vp, pt, sl)
    torch.cuda.synchronize()
    diff = ~((kp == before_k) | (torch.isnan(kp) & torch.isnan(before_k)))
    slots = diff.any(dim=3).any(dim=1).nonzero()   # (page, slot) pairs that changed
    assert len(slots) <= 6
    first = 0
    for b, n in enumerate(d["seq_lens"].tolist()):
        c = (n + 15) // 16
        page = int(d["page_table"][first + (n - 1) // 16])
        assert torch.all(kp[page, :, (n - 1) % 16] == 1)
        first += c


def test_zero_length_sequence_writes_nothing():
    # seq_lens[b] = 0 is outside the precondition (>= 1); the kernel must still
    # leave every slot alone for it rather than write through the table entry
    # before its own (the previous sequence's last page)
    say("kv_append with a zero-length sequence")
    Hkv, D, ps = 2, 128, 16
    lens = torch.tensor([5, 0, 16, 0], dtype=torch.int32)
    pages = [(int(n) + ps - 1) // ps for n in lens]
    npages = sum(pages)
    table = torch.randperm(npages, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    g = torch.Generator().manual_seed(4)
    k_pool = torch.randn((npages, Hkv, ps, D), generator=g).to(torch.bfloat16)
    v_pool = torch.randn((npages, Hkv, ps, D), generator=g).to(torch.bfloat16)
    kn = torch.randn((4, Hkv, D), generator=g).to(torch.bfloat16)
    vn = torch.randn((4, Hkv, D), generator=g).to(torch.bfloat16)
    kp, vp, pt, sl, kn_d, vn_d = cuda(k_pool, v_pool, table, lens, kn, vn)
    attn.kv_append(kn_d, vn_d, kp, vp, pt, sl)
    torch.cuda.synchronize()
    want_k, want_v = k_pool.clone(), v_pool.clone()
    first = 0
    for b, n in enumerate(lens.tolist()):
        if n > 0:
            page = int(table[first + (n - 1) // ps])
            want_k[page, :, (n - 1) % ps] = kn[b]
            want_v[page, :, (n - 1) % ps] = vn[b]
        first += pages[b]
    assert torch.equal(kp.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(vp.cpu().view(torch.int16), want_v.view(torch.int16))
