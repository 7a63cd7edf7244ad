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
sliding-window prefill configurations. ``cpu_baseline`` times the
float64 oracle on a bounded sample of the prefill workload on the host cores.
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


def cpu_baseline(q, k, v, scale, seconds):
    """Time the float64 oracle on whole (batch, head) units of the prefill
    workload until `seconds` have passed; report TFLOP/s on the same
    visible-pair count the GPU figure uses."""
    import numpy as np

    import oracle
    from scaled_dot_product_flash_amd import work

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    B, Hq, Sq, D = qn.shape
    Sk = kn.shape[2]
    units = [(b, h) for b in range(B) for h in range(Hq)]
    np.random.default_rng(0).shuffle(units)
    rows = np.arange(Sq)
    per_unit = work.attention_flops(work.visible_pairs(Sq, Sk, True, 0), D)
    done = 0
    t0 = time.perf_counter()
    for b, h in units:
        out = oracle.attention_rows(qn, kn, vn, b, h, rows, scale, True, 0)
        assert np.isfinite(out).all()
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {
        "value": round(done * per_unit / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(units)} (batch, query head) units of the causal GQA prefill workload, "
                  f"all {Sq} query rows each, float64 numpy, {el:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first; the GPU takes ~50 ms of sustained load to reach its steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    attn.load_library()

    wp, wd = inputs.WORKLOADS[PREFILL], inputs.WORKLOADS[DECODE]
    log("generating inputs")
    q, k, v = inputs.workload_inputs(PREFILL)
    dd = inputs.workload_inputs(DECODE)
    pq, pk, pv = (t.to(dev) for t in (q, k, v))
    po = torch.empty_like(pq)
    dq, dkp, dvp, dpt, dsl = (dd[n].to(dev) for n in ("q", "k_pool", "v_pool", "page_table", "seq_lens"))
    do = torch.empty_like(dq)
    p_scale = 1.0 / math.sqrt(wp["D"])
    d_scale = 1.0 / math.sqrt(wd["D"])
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
        assert torch.isfinite(to.float()).all()
        return w, [e[0].elapsed_time(e[1]) for e in evs]

    other = {}
    for name, reps in (("tiny_f32", 200), ("gpt2_causal", 200), ("swa_16k_w4k", max(args.steps, 20))):
        w, ms = time_prefill(name, reps)
        fl = work.prefill_flops(w["B"], w["Hq"], w["Sq"], w["Sk"], w["D"], w["causal"], w["window"])
        med = sorted(ms)[len(ms) // 2]
        other[name] = {
            "shape": f"B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} Sq=Sk={w['Sq']} D={w['D']} {w['dtype']} "
                     f"causal={w['causal']} window={w['window']}",
            "us_median": round(med * 1e3, 2), "flop_per_call": fl,
            "tflops": round(fl / (med * 1e-3) / 1e12, 3),
            "frac_peak": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if w["dtype"] == "bf16" else None,
        }

    import statistics

    p_flops = work.prefill_flops(wp["B"], wp["Hq"], wp["Sq"], wp["Sk"], wp["D"], True, 0)
    d_bytes = work.decode_kv_bytes(dd["seq_lens"].tolist(), wd["Hkv"], wd["D"], 2)
    p_mean = statistics.fmean(pre_ms)
    d_mean = statistics.fmean(dec_ms)
    p_tflops = p_flops / (p_mean * 1e-3) / 1e12
    d_gbps = d_bytes / (d_mean * 1e-3) / 1e9
    csrc_dir = os.path.join(ROOT, "scaled_dot_product_flash_amd", "csrc")

    out = {
        "metric": METRIC,
        "value": round(p_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
        "prefill": {"ms_mean": round(p_mean, 5), "ms_median": round(statistics.median(pre_ms), 5),
                    "ms_min": round(min(pre_ms), 5), "tflops": round(p_tflops, 3),
                    "frac_peak": round(p_tflops / PEAK_BF16_TFLOPS, 4)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(p_tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": _traffic("prefill_pipe_kernel", os.path.join(csrc_dir, "prefill_bf16.hip")),
        },
        "decode": {
            "value": round(d_gbps, 2),
            "unit": "GB/s",
            "ms_mean": round(d_mean, 5),
            "ms_median": round(statistics.median(dec_ms), 5),
            "ms_min": round(min(dec_ms), 5),
            "roofline": {
                "bound": "hbm",
                "achieved": round(d_gbps, 2),
                "peak": PEAK_HBM_GBPS,
                "unit": "GB/s",
                "frac": round(d_gbps / PEAK_HBM_GBPS, 4),
                "traffic": _traffic("decode_split_kernel", os.path.join(csrc_dir, "decode_paged.hip")),
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
    if not args.no_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s of oracle work)")
        out["cpu_baseline"] = cpu_baseline(q, k, v, p_scale, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
