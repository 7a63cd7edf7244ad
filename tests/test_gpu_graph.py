"""Attention calls captured in a HIP graph (torch.cuda.CUDAGraph).

After a warm-up on the capture stream, which sizes the library's per-stream
workspace so that nothing is allocated while capturing, prefill, paged
prefill, decode, windowed decode and backward calls are captured once and the
graph is replayed three times. Between replays every output is cleared by
eager work and the device synchronised; each replay must reproduce the eager
outputs bit for bit (no memset node is recorded: the kernels write every
output element themselves).
"""

import pytest
import torch

import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def test_graph_replays_match_eager():
    say("graph capture: prefill, paged prefill, decode, windowed decode, backward")
    B, Hq, Hkv, S, D = 2, 8, 2, 333, 128
    q, k, v = (t.cuda() for t in inputs.prefill_inputs(B, Hq, Hkv, S, S, D, "bf16", 77))
    do = torch.randn((B, Hq, S, D), generator=torch.Generator().manual_seed(79)).to(torch.bfloat16).cuda()
    d = inputs.decode_inputs(12, Hq, Hkv, D, 16, 50, 1500, "bf16", seed=78)
    dq1, kp, vp, pt, sl = (d[n].cuda() for n in ("q", "k_pool", "v_pool", "page_table", "seq_lens"))
    qp = torch.randn((12, Hq, 40, D), generator=torch.Generator().manual_seed(80)).to(torch.bfloat16).cuda()
    o_ref, lse = attn.fwd_lse(q, k, v, causal=True)

    outs = {
        "o": torch.empty_like(q),
        "op": torch.empty_like(qp),
        "od": torch.empty_like(dq1),
        "odw": torch.empty_like(dq1),
        "dq": torch.empty_like(q),
        "dk": torch.empty_like(k),
        "dv": torch.empty_like(v),
    }

    def calls():
        attn.fwd(q, k, v, o=outs["o"], causal=True, window=100)
        attn.fwd_paged(qp, kp, vp, pt, sl, o=outs["op"], causal=True)
        attn.decode_paged(dq1, kp, vp, pt, sl, o=outs["od"])
        attn.decode_paged_window(dq1, kp, vp, pt, sl, 300, o=outs["odw"])
        attn.bwd(q, k, v, o_ref, do, lse, causal=True, dq=outs["dq"], dk=outs["dk"], dv=outs["dv"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            calls()
    s.synchronize()
    eager = {n: t.clone() for n, t in outs.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, eager[n]), f"replay {rep}: {n} differs from the eager result"


def test_workspace_under_capture():
    # a graph that captured a decode keeps its workspace after an eager call
    # grows (replaces) the stream's buffer, and a capture that would need a
    # larger workspace is refused instead of allocating
    say("graph capture: workspace retired by growth, growth refused while capturing")
    Hq, Hkv, D = 8, 2, 128
    small = inputs.decode_inputs(4, Hq, Hkv, D, 16, 50, 400, "bf16", seed=81)
    large = inputs.decode_inputs(64, Hq, Hkv, D, 16, 50, 400, "bf16", seed=82)
    names = ("q", "k_pool", "v_pool", "page_table", "seq_lens")
    sd = [small[n].cuda() for n in names]
    ld = [large[n].cuda() for n in names]
    o_small = torch.empty_like(sd[0])
    o_large = torch.empty_like(ld[0])
    s = torch.cuda.Stream()          # a stream of its own: a fresh workspace
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn.decode_paged(*sd, o=o_small)
    s.synchronize()
    want_small = o_small.clone()

    g = torch.cuda.CUDAGraph()
    refused = None
    with torch.cuda.graph(g, stream=s):
        attn.decode_paged(*sd, o=o_small)
        try:
            attn.decode_paged(*ld, o=o_large)   # needs a larger workspace
        except RuntimeError as e:
            refused = str(e)
    torch.cuda.synchronize()
    assert refused is not None and "captured" in refused, refused

    with torch.cuda.stream(s):
        attn.decode_paged(*ld, o=o_large)    # eager: grows the workspace
    s.synchronize()
    want_large = o_large.clone()
    for _ in range(2):
        o_small.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()                           # still the retired buffer
        torch.cuda.synchronize()
        assert torch.equal(o_small, want_small)
    with torch.cuda.stream(s):
        attn.decode_paged(*ld, o=o_large)
    s.synchronize()
    assert torch.equal(o_large, want_large)
