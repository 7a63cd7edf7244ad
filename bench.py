#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

One step = one causal GQA prefill (B=4, Sq=Sk=4096, Hq=32, Hkv=8, D=128, bf16)
followed by one paged GQA decode step (64 sequences, lengths uniform in
[512, 8192], Hq=32, Hkv=8, D=128, page_size 16, bf16). Inputs are seeded
synthetic N(0,1) tensors already resident in HBM.

Printed: ONE JSON line on stdout. ``value`` is prefill attention TFLOP/s
(4·D flop per visible query/key pair) from HIP events around each prefill
launch; the decode step's KV GB/s (every cached K/V byte once) is reported
under ``decode``; ``roofline`` is the prefill kernel against the MI355X dense
bf16 MFMA peak. ``decode_window`` times the sliding-window decode (window
4096) on the same cache, outside the timed steps, as KV GB/s over the
min(len, 4096) most recent tokens of each sequence; ``prefill_lse`` times the
prefill that also returns each row's log-sum-exp; ``prefill_paged`` times a
chunked prefill (512 new tokens per sequence) against a paged cache;
``kv_append`` times the
append of one new token per sequence to the same cache; ``backward`` times the
backward pass (dQ, dK, dV) on the prefill shape at 10·D flop per visible pair;
``other_prefill`` times the float32 128-token, GPT-2-sized causal and 16k
sliding-window prefill configurations. ``cpu_baseline`` times the float64
oracle over the whole prefill workload and the whole decode workload on the
host cores (a pool of single-threaded worker processes, at most 16).
Before the warmup, the step runs back to back for ``--settle-ms`` so that no
timed step sees the clock ramp of an idle GPU; the headline is the median
launch, with mean, standard deviation and minimum beside it. ``counters``
holds what rocprofv3 --pmc reads on a child run of the step: the prefill
kernel's MFMA utilisation (SQ_VALU_MFMA_BUSY_CYCLES over the cycles of its
SIMDs) and the HBM bytes and GB/s of both kernels (FETCH_SIZE and WRITE_SIZE
scaled by what they read for a plain device copy); ``roofline.traffic`` comes
from there (from the committed profile summary when the passes cannot run,
e.g. under ``--no-counters``).
Progress goes to stderr.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s + paged-decode KV GB/s, fraction of MI355X peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PREFILL = "gqa_causal_4k"
DECODE = "paged_decode"
WINDOW = 4096               # sliding-window decode measured beside the step
TRAFFIC_SOURCE = ("profiles/traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE per dispatch, scaled by a plain copy, "
                  "taken on the kernel source whose sha256 it records (null when the source has changed since)")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _kernel_sha256(source_file):
    """SHA-256 over a kernel source followed by every header beside it (the
    work deal and launch arguments live there), in name order."""
    d = os.path.dirname(source_file)
    h = hashlib.sha256()
    for path in [source_file] + sorted(os.path.join(d, n) for n in os.listdir(d) if n.endswith(".h")):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic(kernel_key, source_file):
    """HBM bytes per launch from the committed PMC summary, if the kernel's
    source and headers are unchanged since those counters were taken; else
    None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[kernel_key]
        sha = _kernel_sha256(source_file)
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


# ---- CPU baseline: the float64 oracle in a pool of single-threaded workers ----
# The pool is forked before the GPU is touched, with the inputs already in
# module globals (shared copy-on-write); each worker limits BLAS to one thread.

_CPU = {}


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:
        pass


def _cpu_prefill_unit(bh):
    import numpy as np

    import oracle

    b, h = bh
    c = _CPU["prefill"]
    t0 = time.perf_counter()
    out = oracle.attention_rows(c["q"], c["k"], c["v"], b, h, np.arange(c["q"].shape[2]), c["scale"], True, 0)
    assert np.isfinite(out).all()
    return time.perf_counter() - t0


def _cpu_decode_seq(b):
    import numpy as np

    import oracle

    c = _CPU["decode"]
    first, count = int(c["first"][b]), int(c["count"][b])
    t0 = time.perf_counter()
    out = oracle.decode_paged(c["q"][b:b + 1], c["k_pool"], c["v_pool"], c["page_table"][first:first + count],
                              c["seq_lens"][b:b + 1], c["page_size"], c["scale"])
    assert np.isfinite(out).all()
    return time.perf_counter() - t0


def cpu_workers():
    """Worker count: the host cores this process may run on, at most 16 (one
    GPU's share of a GPU host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_prepare(q, k, v, p_scale, dd, d_scale, page_size):
    """Float32 copies (the exact bf16 values) of both workloads for the oracle
    workers, then the fork of the worker pool."""
    import multiprocessing as mp

    import numpy as np

    _CPU["prefill"] = {"q": q.float().numpy(), "k": k.float().numpy(), "v": v.float().numpy(), "scale": p_scale}
    lens = dd["seq_lens"].numpy().astype(np.int64)
    count = (lens + page_size - 1) // page_size
    _CPU["decode"] = {"q": dd["q"].float().numpy(), "k_pool": dd["k_pool"].float().numpy(),
                      "v_pool": dd["v_pool"].float().numpy(), "page_table": dd["page_table"].numpy(),
                      "seq_lens": dd["seq_lens"].numpy(), "first": np.concatenate([[0], np.cumsum(count)[:-1]]),
                      "count": count, "page_size": page_size, "scale": d_scale}
    n = cpu_workers()
    return mp.get_context("fork").Pool(n, initializer=_cpu_worker_init), n


def cpu_baseline(pool, n, p_flops, d_bytes):
    """Time the float64 oracle over the whole prefill workload (every
    (batch, query head), all query rows) and the whole decode workload (every
    sequence), spread over the worker pool; report TFLOP/s and GB/s on the
    algorithmic counts the GPU figures use."""
    import random

    c = _CPU["prefill"]
    B, Hq = c["q"].shape[:2]
    units = [(b, h) for b in range(B) for h in range(Hq)]
    random.Random(0).shuffle(units)
    pool.map(time.sleep, [0.05] * n)          # every worker started
    t0 = time.perf_counter()
    unit_s = pool.map(_cpu_prefill_unit, units, chunksize=1)
    p_wall = time.perf_counter() - t0
    nseq = len(_CPU["decode"]["seq_lens"])
    seqs = list(range(nseq))
    random.Random(1).shuffle(seqs)
    t0 = time.perf_counter()
    seq_s = pool.map(_cpu_decode_seq, seqs, chunksize=1)
    d_wall = time.perf_counter() - t0
    pool.close()
    pool.join()
    return {
        "value": round(p_flops / p_wall / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": n,
        "kind": "oracle",
        "sample": f"the whole causal GQA prefill workload: all {len(units)} (batch, query head) units, every query "
                  f"row, float64 numpy, {n} single-threaded worker processes, {p_wall:.2f} s wall "
                  f"({sum(unit_s):.1f} s of worker time)",
        "decode": {
            "value": round(d_bytes / d_wall / 1e9, 4),
            "unit": "GB/s",
            "sample": f"the whole paged decode workload: all {nseq} sequences, float64 numpy, {n} single-threaded "
                      f"worker processes, {d_wall:.2f} s wall ({sum(seq_s):.1f} s of worker time)",
        },
    }


# ---- hardware counters: rocprofv3 --pmc over a child run of the step ----
# Two passes (the TCC block holds FETCH_SIZE or WRITE_SIZE, not both). The
# child runs the step's two calls and one plain 256 MiB device copy per step,
# a few times after a short settle; the copy gives each byte counter's scale.

COUNTER_PASSES = (
    ("FETCH_SIZE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"),
    ("WRITE_SIZE",),
)
COUNTER_STEPS = 3
COPY_BYTES = 256 << 20


def _rocprofv3():
    import shutil

    p = shutil.which("rocprofv3")
    if p is None and os.path.exists("/opt/rocm/bin/rocprofv3"):
        p = "/opt/rocm/bin/rocprofv3"
    return p


def _pmc_pass(prof, counters, timeout_s=150):
    """One rocprofv3 --pmc pass over `bench.py --counter-child`; returns
    {kernel name: [per-dispatch {counter: value, "dur_ns": ...}]} in dispatch
    order, or raises RuntimeError."""
    import csv
    import glob
    import shutil
    import signal
    import subprocess
    import tempfile

    d = tempfile.mkdtemp(prefix="attn_pmc_", dir="/tmp")
    cmd = [prof, "--pmc", *counters, "-d", d, "-o", "run", "--output-format", "csv", "--",
           sys.executable, os.path.abspath(__file__), "--counter-child"]
    env = dict(os.environ, TMPDIR="/tmp")
    try:
        proc = subprocess.Popen(cmd, cwd="/tmp", env=env, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE,
                                start_new_session=True)
        try:
            _, err = proc.communicate(timeout=timeout_s)
        except subprocess.TimeoutExpired:
            os.killpg(proc.pid, signal.SIGKILL)
            proc.communicate()
            raise RuntimeError(f"rocprofv3 --pmc {' '.join(counters)}: no result within {timeout_s} s")
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            tail = err.decode(errors="replace").strip().splitlines()[-1:] if err else []
            raise RuntimeError(f"rocprofv3 --pmc {' '.join(counters)} exited {proc.returncode} without a counter "
                               f"file {tail}")
        per = {}
        with open(files[0]) as f:
            for row in csv.DictReader(f):
                rec = per.setdefault(row["Kernel_Name"], {}).setdefault(int(row["Dispatch_Id"]), {})
                rec[row["Counter_Name"]] = float(row["Counter_Value"])
                rec["dur_ns"] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
        return {k: [v[i] for i in sorted(v)] for k, v in per.items()}
    finally:
        shutil.rmtree(d, ignore_errors=True)


def hardware_counters(num_cu):
    """MFMA utilisation of the prefill kernel and HBM bytes of the prefill
    and decode kernels, from rocprofv3 --pmc passes over a child run of the
    step. Byte counters are scaled by what they read for the plain copy."""
    prof = _rocprofv3()
    if prof is None:
        return {"error": "rocprofv3 not found"}
    try:
        passes = [_pmc_pass(prof, c) for c in COUNTER_PASSES]
    except (RuntimeError, OSError, ValueError, KeyError) as e:
        return {"error": str(e)}
    return summarize_counters(passes[0], passes[1], num_cu)


def summarize_counters(fpass, wpass, num_cu):
    """The counters object from the two passes' per-kernel dispatch records
    ({kernel name: [{counter: value, "dur_ns": ns}, ...]})."""

    def last(per, sub, key):
        names = [n for n in per if sub in n]
        if not names:
            raise KeyError(f"no {sub} dispatch")
        name = max(names, key=lambda n: len(per[n]))
        recs = per[name][-COUNTER_STEPS:]
        return name, sum(r[key] for r in recs) / len(recs), sum(r["dur_ns"] for r in recs) / len(recs)

    def copy_scale(per, key):
        recs = [r for n, v in per.items() if "copyBuffer" in n for r in v if r.get(key, 0.0) > 1024.0]
        if not recs:
            raise KeyError("no copy dispatch")
        return (COPY_BYTES / 1024.0) / (sum(r[key] for r in recs) / len(recs))

    try:
        fs, ws = copy_scale(fpass, "FETCH_SIZE"), copy_scale(wpass, "WRITE_SIZE")
        pname, p_fetch, p_dur = last(fpass, "prefill_pipe_kernel", "FETCH_SIZE")
        _, p_write, _ = last(wpass, "prefill_pipe_kernel", "WRITE_SIZE")
        _, busy, _ = last(fpass, "prefill_pipe_kernel", "SQ_VALU_MFMA_BUSY_CYCLES")
        _, nmfma, _ = last(fpass, "prefill_pipe_kernel", "SQ_INSTS_MFMA")
        _, gui, _ = last(fpass, "prefill_pipe_kernel", "GRBM_GUI_ACTIVE")
        sname, s_fetch, s_dur = last(fpass, "decode_split_kernel", "FETCH_SIZE")
        _, s_write, _ = last(wpass, "decode_split_kernel", "WRITE_SIZE")
        mname, m_fetch, m_dur = last(fpass, "decode_merge_kernel", "FETCH_SIZE")
        _, m_write, _ = last(wpass, "decode_merge_kernel", "WRITE_SIZE")
    except (KeyError, ValueError, ZeroDivisionError) as e:
        return {"error": f"counter files incomplete: {e}"}
    cycles = gui / 8.0                      # GRBM_GUI_ACTIVE sums the 8 XCDs
    simds = 4 * num_cu
    p_bytes = p_fetch * 1024 * fs + p_write * 1024 * ws
    d_bytes = (s_fetch + m_fetch) * 1024 * fs + (s_write + m_write) * 1024 * ws
    d_dur = s_dur + m_dur
    return {
        "source": f"rocprofv3 --pmc, passes {[' '.join(c) for c in COUNTER_PASSES]}, over a child run of the "
                  f"step (each: a 300 ms settle, then {COUNTER_STEPS} steps plus a {COPY_BYTES >> 20} MiB device "
                  f"copy); mean of the last {COUNTER_STEPS} dispatches of each kernel",
        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "prefill": {
            "kernel": pname,
            "duration_us": round(p_dur / 1e3, 2),
            "clock_ghz": round(cycles / p_dur, 3),
            "mfma_insts": int(nmfma),
            "mfma_busy_frac": round(busy / (cycles * simds), 4),
            "mfma_busy_frac_at_2p4ghz": round(busy / (p_dur * 2.4 * simds), 4),
            "hbm_fetch_bytes": int(p_fetch * 1024 * fs), "hbm_write_bytes": int(p_write * 1024 * ws),
            "hbm_bytes": int(p_bytes),
        },
        "decode": {
            "kernels": [sname, mname],
            "duration_us": round(d_dur / 1e3, 2),
            "hbm_bytes": int(d_bytes),
            "hbm_gbps": round(d_bytes / d_dur, 2),
            "frac_peak": round(d_bytes / d_dur / PEAK_HBM_GBPS, 4),
        },
    }


def counter_child():
    """The step kernels under the profiler: settle, then COUNTER_STEPS steps,
    each followed by a plain device copy of COPY_BYTES."""
    import torch

    import scaled_dot_product_flash_amd as attn
    from scaled_dot_product_flash_amd import inputs

    wp, wd = inputs.WORKLOADS[PREFILL], inputs.WORKLOADS[DECODE]
    q, k, v = inputs.workload_inputs(PREFILL)
    dd = inputs.workload_inputs(DECODE)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    attn.load_library()
    pq, pk, pv = (t.to(dev) for t in (q, k, v))
    po = torch.empty_like(pq)
    dq, dkp, dvp, dpt, dsl = (dd[n].to(dev) for n in ("q", "k_pool", "v_pool", "page_table", "seq_lens"))
    do = torch.empty_like(dq)
    csrc = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    p_scale, d_scale = 1.0 / math.sqrt(wp["D"]), 1.0 / math.sqrt(wd["D"])

    def step():
        attn.fwd(pq, pk, pv, o=po, scale=p_scale, causal=True, window=0)
        attn.decode_paged(dq, dkp, dvp, dpt, dsl, scale=d_scale, o=do)

    t0 = time.perf_counter()
    while (time.perf_counter() - t0) < 0.3:
        step()
        torch.cuda.synchronize()
    for _ in range(COUNTER_STEPS):
        step()
        cdst.copy_(csrc)
    torch.cuda.synchronize()


def main():
    if "--counter-child" in sys.argv[1:]:
        counter_child()
        return
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first; the GPU takes ~50 ms of sustained load to reach its steady clocks")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed steps run back to back for this long before the warmup, so the GPU reaches its "
                         "sustained clocks before any timed step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-counters", action="store_true",
                    help="skip the rocprofv3 --pmc passes (needed when bench.py itself runs under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="add one plain 256 MiB device copy per step (byte-counter scale for PMC runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (its kernels run on one GPU's "
              "share of the work). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import scaled_dot_product_flash_amd as attn
    from scaled_dot_product_flash_amd import inputs, work

    wp, wd = inputs.WORKLOADS[PREFILL], inputs.WORKLOADS[DECODE]
    log("generating inputs")
    q, k, v = inputs.workload_inputs(PREFILL)
    dd = inputs.workload_inputs(DECODE)
    p_scale = 1.0 / math.sqrt(wp["D"])
    d_scale = 1.0 / math.sqrt(wd["D"])
    pool = None
    if not args.no_cpu_baseline:
        # forked before anything touches the GPU
        pool, n_workers = cpu_prepare(q, k, v, p_scale, dd, d_scale, wd["page_size"])

    if not torch.cuda.is_available():
        if pool is not None:
            pool.terminate()
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    attn.load_library()

    pq, pk, pv = (t.to(dev) for t in (q, k, v))
    po = torch.empty_like(pq)
    dq, dkp, dvp, dpt, dsl = (dd[n].to(dev) for n in ("q", "k_pool", "v_pool", "page_table", "seq_lens"))
    do = torch.empty_like(dq)
    if args.copy_calibration:
        csrc = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        cdst = torch.empty_like(csrc)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        attn.fwd(pq, pk, pv, o=po, scale=p_scale, causal=True, window=0)
        if ev is not None:
            ev[1].record()
        attn.decode_paged(dq, dkp, dvp, dpt, dsl, scale=d_scale, o=do)
        if ev is not None:
            ev[2].record()
        if args.copy_calibration:
            cdst.copy_(csrc)

    # settle: the same step back to back until the GPU has run under load for
    # settle_ms (its clocks take tens of ms of sustained load to level off)
    log(f"settle {args.settle_ms:.0f} ms")
    settle_steps = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= args.settle_ms:
            break
    settle_ms = (time.perf_counter() - t0) * 1e3
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    assert torch.isfinite(po.float()).all() and torch.isfinite(do.float()).all()
    log("timing done")

    # sliding-window decode on the same cache (outside the timed steps)
    dwo = torch.empty_like(dq)
    for _ in range(args.warmup):
        attn.decode_paged_window(dq, dkp, dvp, dpt, dsl, WINDOW, scale=d_scale, o=dwo)
    # every timed loop below enqueues back to back and synchronises once, like
    # the step loop, so the GPU runs under the same sustained load
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        attn.fwd(pq, pk, pv, o=po, scale=p_scale, causal=True, window=0)  # same cache state as a step
        e[0].record()
        attn.decode_paged_window(dq, dkp, dvp, dpt, dsl, WINDOW, scale=d_scale, o=dwo)
        e[1].record()
    torch.cuda.synchronize()
    win_ms = [e[0].elapsed_time(e[1]) for e in ev]
    assert torch.isfinite(dwo.float()).all()

    # prefill that also writes the per-row log-sum-exp (outside the timed steps)
    plse = torch.empty((wp["B"], wp["Hq"], wp["Sq"]), dtype=torch.float32, device=dev)
    lib = attn.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def fwd_lse():
        rc = lib.attn_fwd_lse(pq.data_ptr(), pk.data_ptr(), pv.data_ptr(), po.data_ptr(), plse.data_ptr(),
                              wp["B"], wp["Hq"], wp["Hkv"], wp["Sq"], wp["Sk"], wp["D"], p_scale, 1, 0, stream)
        assert rc == 0, attn.strerror(rc)

    for _ in range(args.warmup):
        fwd_lse()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        fwd_lse()
        e[1].record()
        attn.decode_paged(dq, dkp, dvp, dpt, dsl, scale=d_scale, o=do)  # same load as a step
    torch.cuda.synchronize()
    lse_ms = [e[0].elapsed_time(e[1]) for e in ev]
    assert torch.isfinite(plse).all()

    # chunked prefill against a paged cache (outside the timed steps)
    wc = inputs.WORKLOADS["chunked_prefill_paged"]
    cd = inputs.workload_inputs("chunked_prefill_paged")
    cq, ckp, cvp, cpt, csl = (cd[n].to(dev) for n in ("q", "k_pool", "v_pool", "page_table", "seq_lens"))
    co = torch.empty_like(cq)
    for _ in range(args.warmup):
        attn.fwd_paged(cq, ckp, cvp, cpt, csl, o=co, causal=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        attn.fwd_paged(cq, ckp, cvp, cpt, csl, o=co, causal=True)
        e[1].record()
    torch.cuda.synchronize()
    chunk_ms = [e[0].elapsed_time(e[1]) for e in ev]
    assert torch.isfinite(co.float()).all()
    chunk_flops = sum(work.attention_flops(work.visible_pairs(wc["Sq"], int(n), True, 0), wc["D"]) * wc["Hq"]
                      for n in cd["seq_lens"].tolist())

    # KV append of one new token per sequence (outside the timed steps; it
    # rewrites the last cached token of each sequence)
    kn = torch.randn((wd["nseq"], wd["Hkv"], wd["D"]), device=dev).to(torch.bfloat16)
    vn = torch.randn_like(kn)
    for _ in range(args.warmup):
        attn.kv_append(kn, vn, dkp, dvp, dpt, dsl)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        attn.kv_append(kn, vn, dkp, dvp, dpt, dsl)
        e[1].record()
        attn.decode_paged(dq, dkp, dvp, dpt, dsl, scale=d_scale, o=do)  # the step an append precedes
    torch.cuda.synchronize()
    app_ms = [e[0].elapsed_time(e[1]) for e in ev]

    # backward pass on the prefill shape (outside the timed steps): attn_bwd
    # from q, k, v, o, dO and the forward's lse
    wb = inputs.WORKLOADS["gqa_causal_4k_bwd"]
    bq, bk, bv, bdo = (t.to(dev) for t in inputs.workload_inputs("gqa_causal_4k_bwd"))
    bo, blse = attn.fwd_lse(bq, bk, bv, causal=True)
    bdq, bdk, bdv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
    for _ in range(args.warmup):
        attn.bwd(bq, bk, bv, bo, bdo, blse, causal=True, dq=bdq, dk=bdk, dv=bdv)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        attn.bwd(bq, bk, bv, bo, bdo, blse, causal=True, dq=bdq, dk=bdk, dv=bdv)
        e[1].record()
    torch.cuda.synchronize()
    bwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    assert all(torch.isfinite(t.float()).all() for t in (bdq, bdk, bdv))
    del bq, bk, bv, bdo, bo, blse, bdq, bdk, bdv

    # the other prefill configurations (outside the timed steps): the
    # float32 128-token case (latency), the GPT-2-sized causal case and the
    # 16k sliding-window case, each timed back to back after a warm-up
    def time_prefill(name, reps):
        w = inputs.WORKLOADS[name]
        tq, tk, tv = (t.to(dev) for t in inputs.workload_inputs(name))
        to = torch.empty_like(tq)
        fn = attn.fwd_f32 if w["dtype"] == "f32" else attn.fwd
        for _ in range(reps):
            fn(tq, tk, tv, o=to, causal=w["causal"], window=w["window"])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in evs:
            e[0].record()
            fn(tq, tk, tv, o=to, causal=w["causal"], window=w["window"])
            e[1].record()
        torch.cuda.synchronize()
        # the same calls back to back between two events: a short kernel's
        # launch then overlaps the previous call instead of being timed
        bb = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        bb[0].record()
        for _ in range(reps):
            fn(tq, tk, tv, o=to, causal=w["causal"], window=w["window"])
        bb[1].record()
        torch.cuda.synchronize()
        assert torch.isfinite(to.float()).all()
        return w, [e[0].elapsed_time(e[1]) for e in evs], bb[0].elapsed_time(bb[1]) / reps

    other = {}
    for name, reps in (("tiny_f32", 200), ("gpt2_causal", 200), ("swa_16k_w4k", max(args.steps, 20))):
        w, ms, bb_ms = time_prefill(name, reps)
        fl = work.prefill_flops(w["B"], w["Hq"], w["Sq"], w["Sk"], w["D"], w["causal"], w["window"])
        med = sorted(ms)[len(ms) // 2]
        other[name] = {
            "shape": f"B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} Sq=Sk={w['Sq']} D={w['D']} {w['dtype']} "
                     f"causal={w['causal']} window={w['window']}",
            "us_median": round(med * 1e3, 2), "flop_per_call": fl,
            "tflops": round(fl / (med * 1e-3) / 1e12, 3),
            "frac_peak": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if w["dtype"] == "bf16" else None,
            "us_back_to_back": round(bb_ms * 1e3, 2),
            "tflops_back_to_back": round(fl / (bb_ms * 1e-3) / 1e12, 3),
            "timing": "us_median: events around each call; us_back_to_back: the calls back to back between two "
                      "events, divided by their number",
        }

    import statistics

    p_flops = work.prefill_flops(wp["B"], wp["Hq"], wp["Sq"], wp["Sk"], wp["D"], True, 0)
    d_bytes = work.decode_kv_bytes(dd["seq_lens"].tolist(), wd["Hkv"], wd["D"], 2)
    p_mean, p_med = statistics.fmean(pre_ms), statistics.median(pre_ms)
    d_mean, d_med = statistics.fmean(dec_ms), statistics.median(dec_ms)
    p_std = statistics.stdev(pre_ms) if len(pre_ms) > 1 else 0.0
    d_std = statistics.stdev(dec_ms) if len(dec_ms) > 1 else 0.0
    # headline: the median launch; the roofline uses the mean launch duration
    # (what a kernel trace averages)
    p_tflops = p_flops / (p_med * 1e-3) / 1e12
    d_gbps = d_bytes / (d_med * 1e-3) / 1e9
    p_tflops_mean = p_flops / (p_mean * 1e-3) / 1e12
    d_gbps_mean = d_bytes / (d_mean * 1e-3) / 1e9
    csrc_dir = os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc")

    out = {
        "metric": METRIC,
        "value": round(p_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal GQA prefill B=4 Sq=Sk=4096 Hq=32 Hkv=8 D=128 + paged GQA decode "
                        "64 seqs len~U[512,8192] Hq=32 Hkv=8 D=128 page_size=16",
            "prefill": {"B": wp["B"], "Hq": wp["Hq"], "Hkv": wp["Hkv"], "Sq": wp["Sq"], "Sk": wp["Sk"],
                        "D": wp["D"], "causal": True, "window": 0, "flop_per_call": p_flops},
            "decode": {"seqs": wd["nseq"], "Hq": wd["Hq"], "Hkv": wd["Hkv"], "D": wd["D"],
                       "page_size": wd["page_size"], "tokens": int(dd["seq_lens"].sum()),
                       "kv_bytes_per_call": d_bytes},
            "parallelism": "single GPU",
        },
        "prefill": {"ms_median": round(p_med, 5), "ms_mean": round(p_mean, 5), "ms_std": round(p_std, 5),
                    "ms_min": round(min(pre_ms), 5), "tflops": round(p_tflops, 3),
                    "tflops_at_mean": round(p_tflops_mean, 3), "frac_peak": round(p_tflops / PEAK_BF16_TFLOPS, 4)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(p_tflops_mean, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(p_tflops_mean / PEAK_BF16_TFLOPS, 4),
            "traffic": _traffic("prefill_pipe_kernel", os.path.join(csrc_dir, "prefill_bf16.hip")),
            "achieved_from": "algorithmic flop per launch / mean launch duration (HIP events on the launch stream)",
            "traffic_source": TRAFFIC_SOURCE,
        },
        "decode": {
            "value": round(d_gbps, 2),
            "unit": "GB/s",
            "ms_median": round(d_med, 5),
            "ms_mean": round(d_mean, 5),
            "ms_std": round(d_std, 5),
            "ms_min": round(min(dec_ms), 5),
            "roofline": {
                "bound": "hbm",
                "achieved": round(d_gbps_mean, 2),
                "peak": PEAK_HBM_GBPS,
                "unit": "GB/s",
                "frac": round(d_gbps_mean / PEAK_HBM_GBPS, 4),
                "traffic": _traffic("decode_split_kernel", os.path.join(csrc_dir, "decode_paged.hip")),
                "achieved_from": "KV bytes per call / mean duration of the call (split and merge kernels)",
                "traffic_source": TRAFFIC_SOURCE,
            },
        },
    }
    w_bytes = work.decode_window_kv_bytes(dd["seq_lens"].tolist(), wd["Hkv"], wd["D"], WINDOW, 2)
    w_mean = statistics.fmean(win_ms)
    w_gbps = w_bytes / (w_mean * 1e-3) / 1e9
    out["decode_window"] = {
        "window": WINDOW, "value": round(w_gbps, 2), "unit": "GB/s", "kv_bytes_per_call": w_bytes,
        "ms_mean": round(w_mean, 5), "ms_median": round(statistics.median(win_ms), 5),
        "roofline": {"bound": "hbm", "achieved": round(w_gbps, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(w_gbps / PEAK_HBM_GBPS, 4)},
    }
    l_mean = statistics.fmean(lse_ms)
    out["prefill_lse"] = {"ms_mean": round(l_mean, 5), "tflops": round(p_flops / (l_mean * 1e-3) / 1e12, 3),
                          "frac_peak": round(p_flops / (l_mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    c_mean = statistics.fmean(chunk_ms)
    out["prefill_paged"] = {
        "workload": f"chunked prefill: {wc['nseq']} seqs, {wc['Sq']} new tokens each, cache "
                    f"{wc['len_lo']}..{wc['len_hi']} tokens, Hq={wc['Hq']} Hkv={wc['Hkv']} D={wc['D']} "
                    f"page_size={wc['page_size']}, causal",
        "flop_per_call": chunk_flops, "ms_mean": round(c_mean, 5),
        "tflops": round(chunk_flops / (c_mean * 1e-3) / 1e12, 3),
        "frac_peak": round(chunk_flops / (c_mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    a_bytes = 2 * 2 * wd["nseq"] * wd["Hkv"] * wd["D"] * 2   # k_new, v_new read; two slots written
    a_med = statistics.median(app_ms)
    out["kv_append"] = {
        "us_median": round(a_med * 1e3, 2), "us_mean": round(statistics.fmean(app_ms) * 1e3, 2),
        "bytes_per_call": a_bytes, "GBps": round(a_bytes / (a_med * 1e-3) / 1e9, 2),
        "note": "latency-bound: a few KiB per sequence, one workgroup per sequence",
    }
    b_flops = work.backward_flops(wb["B"], wb["Hq"], wb["Sq"], wb["Sk"], wb["D"], True, 0)
    b_mean = statistics.fmean(bwd_ms)
    b_tflops = b_flops / (b_mean * 1e-3) / 1e12
    out["backward"] = {
        "workload": f"backward of the causal GQA prefill: B={wb['B']} Sq=Sk={wb['Sq']} Hq={wb['Hq']} "
                    f"Hkv={wb['Hkv']} D={wb['D']}",
        "flop_per_call": b_flops, "flop_convention": "10*D per visible pair (2.5x the forward)",
        "ms_mean": round(b_mean, 5), "ms_median": round(statistics.median(bwd_ms), 5),
        "ms_min": round(min(bwd_ms), 5), "tflops": round(b_tflops, 3),
        "frac_peak": round(b_tflops / PEAK_BF16_TFLOPS, 4),
        "kernels": "bwd_dq_kernel then bwd_dkdv_kernel; scores and dP are computed in both (14*D executed)",
    }
    out["other_prefill"] = other
    if args.no_counters:
        out["counters"] = None
    else:
        log("hardware counters: rocprofv3 --pmc passes over a child run of the step")
        hc = hardware_counters(torch.cuda.get_device_properties(dev).multi_processor_count)
        out["counters"] = hc
        if "error" in hc:
            log(f"counters unavailable: {hc['error']}")
        else:
            src = "counters (this run): rocprofv3 FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a plain copy"
            out["roofline"]["traffic"] = hc["prefill"]["hbm_bytes"]
            out["roofline"]["traffic_source"] = src
            out["roofline"]["mfma_busy_frac"] = hc["prefill"]["mfma_busy_frac"]
            out["roofline"]["clock_ghz"] = hc["prefill"]["clock_ghz"]
            out["decode"]["roofline"]["traffic"] = hc["decode"]["hbm_bytes"]
            out["decode"]["roofline"]["traffic_source"] = src
            out["decode"]["roofline"]["counter_gbps"] = hc["decode"]["hbm_gbps"]
    if pool is not None:
        log(f"cpu baseline: the float64 oracle over both workloads, {n_workers} worker processes")
        out["cpu_baseline"] = cpu_baseline(pool, n_workers, p_flops, d_bytes)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
