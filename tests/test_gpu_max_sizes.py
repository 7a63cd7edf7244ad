"""GPU parity at the largest key ranges the C ABI accepts.

The ABI bounds one (batch, kv head) slice of K or V to 2^31 bytes in float32
(Sk * D * 4 < 2^31), so the longest key range is 4194303 tokens at D = 128
and 8388607 at D = 64: byte offsets inside a bf16 slice then reach 2^30 and
inside a float32 slice 2^31 - 512. The prefill (bf16 and float32), the paged
decode (the vector kernel and the MFMA kernel) and the backward run over such
key ranges; sampled query rows, each a softmax over millions of keys, are
compared with the float64 oracle at the usual bars.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import check_bf16, check_f32, check_grad, cuda, f64, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]

# longest key range per head dimension: Sk * D * 4 <= 2^31 - 1
MAX_SK = {D: (2 ** 31 - 1) // (D * 4) for D in (64, 128)}
LSE_BF16_BAR = 2.0 ** -8


def test_prefill_longest_key_range_bf16_d128():
    Sk, Sq = MAX_SK[128], 130
    say(f"prefill bf16 B=1 Hq=2 Hkv=1 Sq={Sq} Sk={Sk} D=128 causal")
    q, k, v = inputs.prefill_inputs(1, 2, 1, Sq, Sk, 128, "bf16", 91)
    scale = 1.0 / math.sqrt(128)
    qd, kd, vd = cuda(q, k, v)
    o, lse = attn.fwd_lse(qd, kd, vd, scale=scale, causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    rows = [0, 1, 63, 64, 127, 128, 129]   # both 128-row work items, the ragged tail
    for h in range(2):
        want = oracle.attention_rows(qf, kf, vf, 0, h, rows, scale, causal=True)
        check_bf16(f64(o[0, h, rows]), want, f"head {h} rows {rows}")
    # the last two rows are a problem of their own under bottom-right causal
    # alignment: the same positions Sk - 2, Sk - 1
    want_l = oracle.attention_lse(qf[:, :, -2:], kf, vf, scale, causal=True)
    assert np.abs(lse[:, :, -2:].double().numpy() - want_l).max() <= LSE_BF16_BAR


def test_prefill_longest_key_range_bf16_d64():
    Sk, Sq = MAX_SK[64], 3
    say(f"prefill bf16 B=1 Hq=2 Hkv=1 Sq={Sq} Sk={Sk} D=64 non-causal")
    q, k, v = inputs.prefill_inputs(1, 2, 1, Sq, Sk, 64, "bf16", 92)
    scale = 1.0 / math.sqrt(64)
    qd, kd, vd = cuda(q, k, v)
    o = attn.fwd(qd, kd, vd, scale=scale, causal=False).cpu()
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    for h in range(2):
        want = oracle.attention_rows(qf, kf, vf, 0, h, list(range(Sq)), scale)
        check_bf16(f64(o[0, h]), want, f"head {h}")


def test_prefill_longest_key_range_f32():
    Sk, Sq = MAX_SK[128], 17
    say(f"prefill f32 B=1 Hq=1 Hkv=1 Sq={Sq} Sk={Sk} D=128 causal")
    q, k, v = inputs.prefill_inputs(1, 1, 1, Sq, Sk, 128, "f32", 93)
    scale = 1.0 / math.sqrt(128)
    qd, kd, vd = cuda(q, k, v)
    o = attn.fwd_f32(qd, kd, vd, scale=scale, causal=True).cpu()
    rows = [0, 1, 15, 16]   # both 16-row work items
    want = oracle.attention_rows(q.numpy(), k.numpy(), v.numpy(), 0, 0, rows, scale, causal=True)
    check_f32(f64(o[0, 0, rows]), want, f"rows {rows}")


def test_decode_longest_sequence():
    # one sequence of the longest key range next to a short one; the last
    # page's unused slot holds NaN. Two query heads per K/V head take the
    # vector kernel, eight the MFMA kernel.
    lens = [MAX_SK[128], 7]
    say(f"decode bf16 seq_lens={lens} Hkv=1 D=128 page_size=256")
    d = inputs.decode_inputs(2, 8, 1, 128, 256, 0, 0, seq_lens=lens, seed=94)
    scale = 1.0 / math.sqrt(128)
    kp, vp, pt, sl = cuda(d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"])
    kf, vf = d["k_pool"].float().numpy(), d["v_pool"].float().numpy()
    for hq in (2, 8):
        q = d["q"][:, :hq].contiguous()
        o = attn.decode_paged(q.cuda(), kp, vp, pt, sl, scale=scale)
        torch.cuda.synchronize()
        want = oracle.decode_paged(f64(q), kf, vf, d["page_table"].numpy(), d["seq_lens"].numpy(), 256, scale)
        check_bf16(f64(o.cpu()), want, f"{hq} query heads")


def test_backward_long_key_range():
    # 2^21 + 77 keys (byte offsets past 2^29 in K and V), 40 query rows
    Sk, Sq = (1 << 21) + 77, 40
    say(f"backward bf16 B=1 Hq=2 Hkv=1 Sq={Sq} Sk={Sk} D=128 causal")
    q, k, v, do = inputs.backward_inputs(1, 2, 1, Sq, Sk, 128, seed=95)
    scale = 1.0 / math.sqrt(128)
    qd, kd, vd, dod = cuda(q, k, v, do)
    o, lse = attn.fwd_lse(qd, kd, vd, scale=scale, causal=True)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    wq, wk, wv = oracle.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, causal=True)
    check_grad(f64(dq), wq, "dq")
    check_grad(f64(dk), wk, "dk")
    check_grad(f64(dv), wv, "dv")
