"""GPU parity at the element-count and grid limits, through the degenerate
case of a single visible key.

With one visible key the softmax weight is exactly 1 and the output is that
key's value row, "a single key returns its V" (one of the oracle's pins):
the kernels reach it exactly in bf16 (the weight exp2 of a rounding error
rounds to 1.0, the row sum is that 1.0, and V is a bf16 value), so every
output element is compared bit for bit on the GPU, and sampled rows against
the oracle as well.

* prefill: a query tensor of more than 2^32 elements (1024 query heads x
  32769 rows x 128), so element and byte offsets of Q, O and the
  log-sum-exp pass 2^32;
* decode: B = 65535 sequences, the largest batch the ABI accepts, at
  B * Hq = 2^24 - 256 on the MFMA kernel and with one head per K/V head on
  the vector kernel; one cached token each, the other slots of its page NaN.

Inputs are drawn on the GPU from seeded generators.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from gpu_util import check_bf16, check_f32, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _randn(shape, g, dtype):
    return torch.randn(shape, device="cuda", generator=g, dtype=torch.float32).to(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_more_than_2_32_query_elements(dtype):
    B, Hq, Hkv, Sq, Sk, D = 1, 1024, 8, 32769, 1, 128
    assert B * Hq * Sq * D > 2 ** 32
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"prefill {dtype} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} D={D} non-causal (one key)")
    g = torch.Generator(device="cuda").manual_seed(96)
    q = _randn((B, Hq, Sq, D), g, td)
    k = _randn((B, Hkv, Sk, D), g, td)
    v = _randn((B, Hkv, Sk, D), g, td)
    scale = 1.0 / math.sqrt(D)
    fn = attn.fwd_lse if dtype == "bf16" else attn.fwd_f32_lse
    o, lse = fn(q, k, v, scale=scale)
    torch.cuda.synchronize()
    G = Hq // Hkv
    worst = 0.0
    for h in range(Hq):
        want = v[0, h // G, 0][None, :].expand(Sq, D)
        if dtype == "bf16":
            assert torch.equal(o[0, h], want), f"head {h}"
        else:
            worst = max(worst, (o[0, h] - want).abs().max().item())
    # float32 keeps the weight's rounding error (exp2 of it is 1 + 2^-23 at
    # most), which the division by the same row sum takes out again up to a
    # rounding of each element
    assert worst <= 1e-6 * max(1.0, v.abs().max().item())
    # sampled (head, row) pairs against the oracle's output and log-sum-exp;
    # with a single key every row is a problem of its own, so the rows are
    # handed over on their own
    rows = [0, 255, 256, Sq - 1]
    for h in (0, 7, 8, 513, 1023):
        qs = q[:, h:h + 1, rows].float().cpu().numpy()
        ks = k[:, h // G:h // G + 1].float().cpu().numpy()
        vs = v[:, h // G:h // G + 1].float().cpu().numpy()
        want_o = oracle.attention_rows(qs, ks, vs, 0, 0, list(range(len(rows))), scale)
        (check_bf16 if dtype == "bf16" else check_f32)(f64(o[0, h, rows].float().cpu()), want_o, f"head {h}")
        want_l = oracle.attention_lse(qs, ks, vs, scale)
        got_l = lse[0, h, rows].double().cpu().numpy()
        assert np.abs(got_l - want_l[0, 0]).max() <= (2.0 ** -8 if dtype == "bf16" else 1e-5)
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("Hq,Hkv", [(256, 16), (2, 2)])
def test_decode_largest_batch(Hq, Hkv):
    # (256, 16): sixteen heads per K/V head, the MFMA kernel, B * Hq =
    # 2^24 - 256; (2, 2): one head per K/V head, the vector kernel
    B, D, ps = 65535, 128, 8
    say(f"decode bf16 B={B} Hq={Hq} Hkv={Hkv} D={D} page_size={ps}, one cached token each")
    g = torch.Generator(device="cuda").manual_seed(97 + Hq)
    q = _randn((B, Hq, D), g, torch.bfloat16)
    k_pool = _randn((B, Hkv, ps, D), g, torch.bfloat16)
    v_pool = _randn((B, Hkv, ps, D), g, torch.bfloat16)
    k_pool[:, :, 1:, :] = float("nan")
    v_pool[:, :, 1:, :] = float("nan")
    table = torch.randperm(B, device="cuda", generator=g).to(torch.int32)
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    o = attn.decode_paged(q, k_pool, v_pool, table, lens, scale=1.0 / math.sqrt(D))
    torch.cuda.synchronize()
    want = v_pool[table.long(), :, 0, :].repeat_interleave(Hq // Hkv, 1)
    assert torch.equal(o, want)
    # a few sequences through the oracle, their pages in a pool of their own
    pick = [0, 1, 4097, B - 1]
    pages = table[pick].long()
    got = f64(o[pick].float().cpu())
    want_o = oracle.decode_paged(f64(q[pick].float().cpu()), k_pool[pages].float().cpu().numpy(),
                                 v_pool[pages].float().cpu().numpy(), np.arange(len(pick), dtype=np.int32),
                                 np.ones(len(pick), dtype=np.int32), ps, 1.0 / math.sqrt(D))
    check_bf16(got, want_o, "sampled sequences")
    del q, k_pool, v_pool, o, want
    torch.cuda.empty_cache()
