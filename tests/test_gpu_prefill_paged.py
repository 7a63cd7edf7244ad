"""GPU parity of attn_fwd_paged (prefill of the newest Sq tokens of each
sequence against a paged cache) with the float64 oracle.

Pools are built by the seeded decode generator: a random permutation of
pages, NaN in every slot past a sequence's length.
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


def _case(lens, Hq, Hkv, Sq, ps, seed, D):
    d = inputs.decode_inputs(len(lens), Hq, Hkv, D, ps, 0, 0, "bf16", seed=seed, seq_lens=lens)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((len(lens), Hq, Sq, D), generator=g).to(torch.bfloat16)
    return q, d


def _oracle(q, d, scale, causal, window):
    return oracle.prefill_paged(f64(q), d["k_pool"].float().numpy(), d["v_pool"].float().numpy(),
                                d["page_table"].numpy(), d["seq_lens"].numpy(), d["k_pool"].shape[2],
                                scale, causal, window)


CASES = [
    # lens, Hq, Hkv, Sq, page_size, causal, window, D
    ([300, 64, 129], 8, 2, 64, 16, True, 0, 128),
    ([1000, 700], 8, 2, 256, 16, True, 0, 128),       # chunked prefill: Sq < len
    ([256, 257], 4, 4, 256, 32, True, 0, 128),        # the whole sequence is new
    ([500, 80], 8, 1, 80, 8, True, 37, 128),          # sliding window, MQA
    ([200, 333, 17], 4, 2, 17, 256, False, 0, 128),   # non-causal
    ([4096, 2500, 3000, 1], 32, 8, 1, 16, True, 0, 128),   # Sq = 1: a decode step
    ([130, 5000], 16, 4, 130, 64, True, 1000, 128),
    ([300, 64, 129], 8, 2, 64, 16, True, 0, 64),      # D = 64: four waves, eight rows per DMA slot
    ([1000, 700], 12, 12, 256, 8, True, 0, 64),
    ([500, 80], 8, 1, 80, 32, True, 37, 64),
    ([200, 333, 17], 4, 2, 17, 256, False, 0, 64),
    ([2000, 1], 8, 2, 1, 16, True, 0, 64),
    # more (sequence, kv head) groups than XCDs: groups dealt in snake order,
    # 15 chunks leave the second round one short
    ([900, 50, 400, 1200, 47], 6, 3, 40, 16, True, 0, 128),
    # more sequences than the in-kernel longest-first ranking covers (512 for
    # eight waves, 256 for four waves as at D = 64): slots keep batch order
    ([int(x) for x in np.random.default_rng(7).integers(3, 71, 600)], 8, 2, 3, 8, True, 0, 128),
    ([int(x) for x in np.random.default_rng(8).integers(3, 301, 301)], 4, 4, 3, 16, True, 5, 64),
]


@pytest.mark.parametrize("case", CASES)
def test_paged_prefill_cases(case):
    lens, Hq, Hkv, Sq, ps, causal, window, D = case
    say(f"paged prefill {(lens if len(lens) < 8 else f'{len(lens)} seqs'), Hq, Hkv, Sq, ps, causal, window, D}")
    q, d = _case(lens, Hq, Hkv, Sq, ps, seed=sum(lens) % 997 + Sq, D=D)
    scale = 1.0 / math.sqrt(D)
    qd, kp, vp, pt, sl = cuda(q, d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"])
    o, lse = attn.fwd_paged(qd, kp, vp, pt, sl, scale=scale, causal=causal, window=window, lse=True)
    torch.cuda.synchronize()
    check_bf16(f64(o.cpu()), _oracle(q, d, scale, causal, window), f"{len(lens)} seqs, Sq={Sq}, D={D}")
    # log-sum-exp of the same rows, bar of the bf16 path (see test_gpu_prefill)
    want_lse = np.stack([oracle.attention_lse(
        f64(q[b:b + 1]),
        oracle.gather_sequence(d["k_pool"].float().numpy(), d["page_table"].numpy(), d["seq_lens"].numpy(), ps, b)[None],
        oracle.gather_sequence(d["v_pool"].float().numpy(), d["page_table"].numpy(), d["seq_lens"].numpy(), ps, b)[None],
        scale, causal, window)[0] for b in range(len(lens))])
    assert np.abs(f64(lse.cpu()) - want_lse).max() <= 2.0 ** -8


@pytest.mark.parametrize("D", [128, 64])
def test_paged_prefill_equals_contiguous_bit_exact(D):
    # same K/V, laid out in pages or contiguously: the same arithmetic
    B, Hq, Hkv, S, ps = 2, 8, 2, 700, 16
    say(f"paged prefill bit-exact D={D}")
    q, k, v = inputs.prefill_inputs(B, Hq, Hkv, S, S, D, "bf16", 45)
    n_pages = (S + ps - 1) // ps
    perm = torch.randperm(B * n_pages, generator=torch.Generator().manual_seed(3))
    kp = torch.full((B * n_pages, Hkv, ps, D), float("nan"), dtype=torch.bfloat16)
    vp = kp.clone()
    for b in range(B):
        for p in range(n_pages):
            t0, t1 = p * ps, min(S, (p + 1) * ps)
            kp[perm[b * n_pages + p], :, :t1 - t0] = k[b, :, t0:t1]
            vp[perm[b * n_pages + p], :, :t1 - t0] = v[b, :, t0:t1]
    table = perm.to(torch.int32)
    sl = torch.full((B,), S, dtype=torch.int32)
    for Sq, window in ((S, 0), (300, 0), (300, 50)):
        qq = q[:, :, S - Sq:].contiguous()
        qd, kd, vd, kpd, vpd, ptd, sld = cuda(qq, k, v, kp, vp, table, sl)
        paged = attn.fwd_paged(qd, kpd, vpd, ptd, sld, causal=True, window=window)
        cont = attn.fwd(qd, kd, vd, causal=True, window=window)
        torch.cuda.synchronize()
        assert torch.equal(paged, cont), (Sq, window)
