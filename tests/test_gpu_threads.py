"""Concurrent calls from several host threads, each on its own stream.

The decode and the backward take their workspace per (device, stream) from
the library, under a lock held until the call's kernels are enqueued; a
larger request retires the old buffer instead of freeing it. Four threads,
each with its own stream, loop over problems of different sizes (so a
stream's workspace grows while other threads are mid-call) and every result
must equal, bit for bit, the same call made alone on the default stream
(both calls are deterministic: the split counts and the backward's order of
summation depend only on the shapes).
"""

import math
import threading

import pytest
import torch

import scaled_dot_product_flash_amd as attn
from scaled_dot_product_flash_amd import inputs
from gpu_util import needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _decode_problem(nseq, Hq, Hkv, D, ps, lo, hi, seed):
    d = inputs.decode_inputs(nseq, Hq, Hkv, D, ps, lo, hi, seed=seed)
    d = {k: v.cuda() for k, v in d.items()}
    scale = 1.0 / math.sqrt(D)

    def run(o=None):
        return attn.decode_paged(d["q"], d["k_pool"], d["v_pool"], d["page_table"], d["seq_lens"], scale=scale, o=o)
    return run


def _backward_problem(B, Hq, Hkv, S, D, seed):
    q, k, v, do = (t.cuda() for t in inputs.backward_inputs(B, Hq, Hkv, S, S, D, seed=seed))
    scale = 1.0 / math.sqrt(D)
    o, lse = attn.fwd_lse(q, k, v, scale=scale, causal=True)

    def run(out=None):
        out = out or (None, None, None)
        return attn.bwd(q, k, v, o, do, lse, scale=scale, causal=True, dq=out[0], dk=out[1], dv=out[2])
    return run


def test_threads_on_own_streams_match_single_calls():
    say("threads: 4 host threads x own streams, decode and backward, growing workspaces")
    problems = [
        ("decode", _decode_problem(8, 32, 8, 128, 16, 100, 900, 11)),
        ("decode", _decode_problem(64, 32, 8, 128, 16, 512, 4096, 12)),   # larger workspace
        ("decode", _decode_problem(5, 16, 1, 64, 32, 50, 3000, 13)),      # MFMA kernel
        ("backward", _backward_problem(1, 8, 2, 700, 128, 14)),
        ("backward", _backward_problem(2, 4, 4, 300, 64, 15)),
    ]
    # references: each call alone on the default stream
    refs = []
    for kind, run in problems:
        r = run()
        refs.append([t.clone() for t in r] if kind == "backward" else r.clone())
    torch.cuda.synchronize()
    attn.release()   # every stream starts with no workspace, so the first calls grow it

    failures = []
    lock = threading.Lock()

    def worker(tid):
        s = torch.cuda.Stream()
        order = [(tid + i) % len(problems) for i in range(len(problems))]
        try:
            with torch.cuda.stream(s):
                for it in range(12):
                    for p in order[::1 if it % 2 == 0 else -1]:
                        kind, run = problems[p]
                        got = run()
                        s.synchronize()
                        want = refs[p]
                        same = all(torch.equal(a, b) for a, b in zip(got, want)) if kind == "backward" \
                            else torch.equal(got, want)
                        if not same:
                            with lock:
                                failures.append((tid, it, p))
        except Exception as e:   # noqa: BLE001 - reported below
            with lock:
                failures.append((tid, "raised", repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=600)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not failures, failures[:5]
