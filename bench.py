"""Benchmark of the frequency-ranked drafter head on one MI355X.

A step is one draft-head call (logits over the kept rows, subset softmax,
top-k, remap: one kernel) on the LLaMA-3-8B drafter head shape: d = 4096,
V = 128256 trimmed to V_high = 32768, M = 1 draft row, k = 10. The kept
vocabulary and W_trim come from the same run's GPU preparation (count 1e8
seeded Zipf ids, select, gather), which is timed too and reported under
"prep"; "pipeline" is one pass of every step, preparation included.

Inputs are resident in HBM before timing starts. W_trim (256 MiB) is about
the size of the 256 MB Infinity Cache, so timed calls rotate over copies
totalling at least 1 GiB ("cold", the reported value); a single resident
copy is reported as "warm". The roofline object divides the algorithmic
bytes of one call by the average call time over the timed region, taken
with HIP events on the stream the kernel runs on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--M M] [--sweep] [--no-cpu] [--only-head [--sample]] [--calib-copy]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak, TFLOP/s
METRIC = "draft-head calls/s & µs/call (d=4096,V_high=32k,M=1); % of peak HBM GB/s"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def head_bytes(V_high, d, M, k):
    """Algorithmic bytes of one draft-head call: W_trim, h, outputs."""
    return 2 * V_high * d + 2 * M * d + 8 * M * k


def time_calls(fn, n, torch):
    """Total ms of n back-to-back calls, events around the region."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for i in range(n):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e)


def per_launch_us(fn, n, torch):
    """Average µs of single launches, each bracketed by its own events."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return 1000.0 * statistics.mean(a.elapsed_time(b) for a, b in evs)


def host_call_us(fn, n, torch):
    """Host wall-clock of the API call itself (argument checks, marshalling,
    the kernel launches; no wait for the GPU), and of one call followed by a
    device synchronisation (the latency a caller that needs the result at
    once sees), each the median over n calls."""
    call, sync = [], []
    torch.cuda.synchronize()
    for i in range(n):
        a = time.perf_counter()
        fn(i)
        b = time.perf_counter()
        torch.cuda.synchronize()
        c = time.perf_counter()
        call.append(b - a)
        sync.append(c - a)
    return 1e6 * statistics.median(call), 1e6 * statistics.median(sync)


def median_us(fn, reps, torch):
    ts = []
    for _ in range(reps):
        ts.append(1000.0 * time_calls(lambda i: fn(), 1, torch))
    return statistics.median(ts)


def head_kernels(M, V_high):
    """The kernels one draft-head call launches (the library's dispatch)."""
    tiles = (V_high + 63) // 64
    if M == 1 or (M == 2 and (tiles + 1) // 2 < 256):
        return "head_gemv_kernel"
    if M > 32 or tiles >= 256:
        return "head_gemm_kernel + tree_merge_kernel"
    return "head_mfma_kernel + tree_merge_kernel"


def recorded_traffic():
    """HBM bytes per launch of the head kernel from the committed counter
    summary, or None if the kernel sources changed since it was taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "head_gemv_llama3_8b_m1.md")
    if not os.path.exists(prof):
        return None
    fields = {}
    for line in open(prof):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256"):
            key, val = line.split(":", 1)
            fields[key] = val.strip()
    h = hashlib.sha256()
    for f in ("head.hip", "vt_device.hpp", "vt_internal.hpp"):
        h.update(open(os.path.join(ROOT, "drafter_lm_head_amd", "csrc", f), "rb").read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_info():
    """(usable host cores, CPU model string)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), model


def cpu_baseline(h, Wt, t2f, k, budget_s=8.0):
    """The unmodified oracle's full draft-head call on the host cores: with
    every OpenMP thread it uses by default and with one thread."""
    import oracle
    oracle.draft_head(h[:1], Wt[:64], t2f[:64], 1)      # load + page in
    nproc, model = cpu_info()

    def run(budget):
        ts, t0 = [], time.perf_counter()
        while True:
            a = time.perf_counter()
            oracle.draft_head(h, Wt, t2f, k)
            ts.append(time.perf_counter() - a)
            if time.perf_counter() - t0 >= budget and len(ts) >= 3:
                break
        return len(ts), sum(ts), statistics.median(ts)

    t_all = oracle.threads()
    n, el, med = run(budget_s)
    oracle.set_threads(1)
    n1, el1, med1 = run(budget_s)
    oracle.set_threads(t_all)
    return {"value": n / el, "unit": "calls/s", "cores": t_all, "kind": "oracle",
            "sample": f"{n} full draft-head calls (fp64 C oracle, OpenMP over rows, {t_all} "
                      f"threads) on the same inputs, {el:.1f} s",
            "median_ms_per_call": round(1000 * med, 3),
            "t1": {"value": n1 / el1, "unit": "calls/s", "cores": 1,
                   "median_ms_per_call": round(1000 * med1, 3),
                   "sample": f"{n1} calls with one thread, {el1:.1f} s"},
            "nproc": nproc, "cpu_model": model}


def interleaved_us(fa, fb, n, rounds, torch):
    """Median µs per call of two call sequences timed in alternating batches."""
    ta, tb = [], []
    for _ in range(rounds):
        ta.append(1000.0 * time_calls(fa, n, torch) / n)
        tb.append(1000.0 * time_calls(fb, n, torch) / n)
    return statistics.median(ta), statistics.median(tb)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only-head", action="store_true",
                    help="time only the cold draft-head steps (for profiler runs)")
    ap.add_argument("--sample", action="store_true",
                    help="with --only-head: time vt_draft_sample (one draw per row) instead")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the draft head is measured on one "
              "MI355X; it has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import drafter_lm_head_amd as dlh
    import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    if args.M is not None:
        w = w.replace(M=args.M)
    log(f"workload {w}")

    # ---------------------------------------------------------- inputs
    t0 = time.perf_counter()
    ids_h = synth.make_ids(w)
    W_h = synth.make_weights(w)
    h_h = synth.make_hidden(w)
    log(f"inputs drawn in {time.perf_counter() - t0:.1f} s")
    ids = torch.from_numpy(ids_h).to(dev)
    W = torch.from_numpy(W_h.view(np.int16)).to(dev)
    h = torch.from_numpy(h_h.view(np.int16)).to(dev)
    torch.cuda.synchronize()

    # ------------------------------------------------------------ prep
    counts, n_inv = dlh.vt_count_freq(ids, w.V)
    t2f, f2t, sel, tot = dlh.vt_select_vocab(counts, w.V_high)
    Wt = dlh.vt_gather_head(W, t2f)
    torch.cuda.synchronize()
    cov = dlh.coverage(sel, tot)
    reps = 1 if args.only_head else 7
    us_count = median_us(lambda: dlh.vt_count_freq(ids, w.V, counts=counts, n_invalid=n_inv), reps, torch)
    us_select = median_us(lambda: dlh.vt_select_vocab(counts, w.V_high), reps, torch)
    us_gather = median_us(lambda: dlh.vt_gather_head(W, t2f, out=Wt), reps, torch)
    order_full, _, _, _ = dlh.vt_select_vocab(counts, w.V)
    us_cov = median_us(lambda: dlh.vt_coverage_curve(counts, order_full, 0.9), reps, torch)
    _, _, vh90 = dlh.vt_coverage_curve(counts, order_full, 0.9)
    v_high_90 = int(vh90.item())
    log(f"prep: count {us_count:.1f} us, select {us_select:.1f} us, gather {us_gather:.1f} us, "
        f"coverage {cov:.4f}")

    # --------------------------------------------------- draft-head setup
    M, d, k, V_high = w.M, w.d, w.k, w.V_high
    wt_bytes = 2 * V_high * d
    R = max(1, math.ceil((1 << 30) / wt_bytes))
    copies = [Wt] + [Wt.clone() for _ in range(R - 1)]
    full_ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    probs = torch.empty((M, k), dtype=torch.float32, device=dev)
    ws = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, k), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def cold(i):
        dlh.vt_draft_head(h, copies[i % R], t2f, k, full_ids=full_ids, probs=probs, ws=ws)

    def warm(i):
        dlh.vt_draft_head(h, Wt, t2f, k, full_ids=full_ids, probs=probs, ws=ws)

    kk = k
    if args.only_head and args.sample:
        # The draw instead of top-k (same contraction, per-tile Gumbel-max
        # draws, one output per row), a new offset per call.
        kk = 1
        s_ws = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, 1), dtype=torch.uint8,
                           device=dev)
        s_out = (torch.empty(M, dtype=torch.int32, device=dev),
                 torch.empty(M, dtype=torch.float32, device=dev))

        def cold(i):
            dlh.vt_draft_sample(h, copies[i % R], t2f, 2024, i, full_ids=s_out[0],
                                probs=s_out[1], ws=s_ws)
    for i in range(args.warmup):
        cold(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} cold steps over {R} W_trim copies")
    ms_total = time_calls(cold, args.steps, torch)
    ms_step = ms_total / args.steps
    value = 1000.0 / ms_step
    nb = head_bytes(V_high, d, M, kk)
    # Roofline: algorithmic bytes over the kernel's average duration in the
    # timed region (events on the stream the kernel runs on).
    achieved = nb / (ms_step * 1e-3) / 1e9
    log(f"cold: {ms_step * 1000:.2f} us/step, {achieved:.0f} GB/s")
    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 10 x 256 MiB")
        del src, dst
    if args.only_head:
        print(json.dumps({"metric": METRIC, "value": round(value, 1), "unit": "calls/s",
                          "ms_per_step": round(ms_step, 6), "steps": args.steps,
                          "GB_per_s": round(achieved, 1), "draw": bool(args.sample)}),
              flush=True)
        return
    n_launch = min(args.steps, 1000)
    us_launch = per_launch_us(cold, n_launch, torch)
    us_host_call, us_host_sync = host_call_us(cold, n_launch, torch)
    ms_warm = time_calls(warm, args.steps, torch) / args.steps
    log(f"warm: {ms_warm * 1000:.2f} us/step; single launches bracketed by events: {us_launch:.2f} us")

    # the pages' own draft step: one multinomial draw per row (Gumbel-max),
    # cold, a new offset per call
    s_ids = torch.empty(M, dtype=torch.int32, device=dev)
    s_p = torch.empty(M, dtype=torch.float32, device=dev)
    ws_s = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, 1), dtype=torch.uint8,
                       device=dev)

    def cold_sample(i):
        dlh.vt_draft_sample(h, copies[i % R], t2f, 2024, i, full_ids=s_ids, probs=s_p, ws=ws_s)
    for i in range(50):
        cold_sample(i)
    ms_sample = time_calls(cold_sample, args.steps, torch) / args.steps
    log(f"sample (cold): {ms_sample * 1000:.2f} us/step")

    # practical ceiling: a plain streaming read of the same W_trim copies
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    read = lambda i: dlh.vt_stream_read(copies[i % R], sink)
    for i in range(50):
        read(i)
    us_read = 1000.0 * time_calls(read, args.steps, torch) / args.steps
    log(f"streaming read of W_trim (cold): {us_read:.2f} us/call")

    # the remap's cost: the same call returning trimmed indices, interleaved
    t_ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    t_p = torch.empty((M, k), dtype=torch.float32, device=dev)
    ws_t = torch.zeros(dlh.vt_draft_head_workspace_size(M, V_high, d, k), dtype=torch.uint8,
                       device=dev)
    trimmed = lambda i: dlh.vt_draft_head_trimmed(h, copies[i % R], k, trimmed_ids=t_ids,
                                                  probs=t_p, ws=ws_t)
    for i in range(50):
        trimmed(i)
    us_remap, us_noremap = interleaved_us(cold, trimmed, max(200, args.steps // 4), 5, torch)
    log(f"remap: {us_remap:.2f} us with, {us_noremap:.2f} us without")

    # the same cold calls replayed from a captured graph (no per-call launch)
    n_graph = 4 * R
    gstream = torch.cuda.Stream()
    gstream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gstream):
        for i in range(n_graph):
            cold(i)
    torch.cuda.current_stream().wait_stream(gstream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_graph):
            cold(i)
    graph.replay()
    reps = max(1, args.steps // n_graph)
    us_graph = 1000.0 * time_calls(lambda i: graph.replay(), reps, torch) / (reps * n_graph)
    log(f"graph replay: {us_graph:.2f} us/call")

    # pipeline: one pass of every step (count, select, gather, draft head)
    def pipeline():
        dlh.vt_count_freq(ids, w.V, counts=counts, n_invalid=n_inv)
        dlh.vt_select_vocab(counts, w.V_high)
        dlh.vt_gather_head(W, t2f, out=Wt)
        dlh.vt_draft_head(h, Wt, t2f, k, full_ids=full_ids, probs=probs, ws=ws)
    us_pipe = median_us(pipeline, 5, torch)

    # untrimmed head: the whole [V, d] head with the identity map
    ident = torch.arange(w.V, dtype=torch.int32, device=dev)
    ws_u = torch.zeros(dlh.vt_draft_head_workspace_size(M, w.V, d, k), dtype=torch.uint8, device=dev)
    fu = lambda i: dlh.vt_draft_head(h, W, ident, k, full_ids=full_ids, probs=probs, ws=ws_u)
    for i in range(20):
        fu(i)
    n_u = max(50, args.steps // 4)
    us_untrim = 1000.0 * time_calls(fu, n_u, torch) / n_u
    log(f"untrimmed V={w.V}: {us_untrim:.2f} us/call")

    sweep = None
    if args.sweep:
        sweep = []
        for vh in synth.SWEEP_V_HIGH:
            t2f_s, _, _, _ = dlh.vt_select_vocab(counts, vh)
            wts = dlh.vt_gather_head(W, t2f_s) if vh < w.V else W
            Rs = max(1, math.ceil((1 << 30) / (2 * vh * d)))
            cs = [wts] + [wts.clone() for _ in range(Rs - 1)]
            wss = torch.zeros(dlh.vt_draft_head_workspace_size(M, vh, d, k), dtype=torch.uint8, device=dev)
            f = lambda i: dlh.vt_draft_head(h, cs[i % Rs], t2f_s, k, full_ids=full_ids, probs=probs, ws=wss)
            for i in range(50):
                f(i)
            us = 1000.0 * time_calls(f, 1000, torch) / 1000
            gbs = head_bytes(vh, d, M, k) / (us * 1e-6) / 1e9
            sweep.append({"V_high": vh, "us_per_call": round(us, 3), "GB_per_s": round(gbs, 1),
                          "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
            log(f"sweep V_high={vh}: {us:.2f} us, {gbs:.0f} GB/s")
            del cs, wts, wss

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(h_h, Wt.view(torch.int16).cpu().numpy().view(np.uint16),
                           t2f.cpu().numpy(), k)

    prep_bytes_count = 4 * w.n_ids + 4 * w.V
    prep_bytes_gather = 2 * 2 * V_high * d + 4 * V_high
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} drafter head (frequency-ranked trim)", "d": d, "V": w.V,
                   "V_high": V_high, "M": M, "k": k, "ids": w.n_ids, "zipf_s": w.zipf_s,
                   "parallelism": "none (1 GPU)", "protocol": f"cold: rotate {R} W_trim copies"},
        "us_per_call": round(ms_step * 1000, 3),
        "hbm_frac": round(nb / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic() if (w.name == "llama3_8b" and M == 1) else None,
                     "kernel": head_kernels(M, V_high),
                     "bytes_per_launch": nb,
                     "us_per_launch": round(ms_step * 1000, 3),
                     "us_single_launch_events": round(us_launch, 3)},
        "cpu_baseline": cpu,
        "ceiling": {"what": "vt_stream_read: plain 16-byte non-temporal streaming read of the "
                            "same W_trim copies (cold), the practical bandwidth ceiling",
                    "bytes_per_call": wt_bytes, "us_per_call": round(us_read, 3),
                    "GB_per_s": round(wt_bytes / (us_read * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(wt_bytes / (us_read * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "head_over_ceiling": round(ms_step * 1000 / us_read, 4)},
        "remap": {"what": "vt_draft_head (full ids through t2f) against vt_draft_head_trimmed "
                          "(trimmed indices), interleaved, cold",
                  "us_with_remap": round(us_remap, 3), "us_without_remap": round(us_noremap, 3),
                  "overhead_frac": round((us_remap - us_noremap) / us_noremap, 5)},
        "host": {"what": "host wall-clock per vt_draft_head call through the binding, launch "
                         "included (median); and the same call followed by a device "
                         "synchronisation",
                 "us_per_api_call": round(us_host_call, 3),
                 "us_call_to_result": round(us_host_sync, 3)},
        "graph": {"what": f"{n_graph} cold calls captured in one graph, replayed",
                  "us_per_call": round(us_graph, 3),
                  "GB_per_s": round(nb / (us_graph * 1e-6) / 1e9, 1)},
        "warm": {"us_per_call": round(ms_warm * 1000, 3),
                 "GB_per_s": round(nb / (ms_warm * 1e-3) / 1e9, 1)},
        "sample": {"us_per_call": round(ms_sample * 1000, 3),
                   "GB_per_s": round(head_bytes(V_high, d, M, 1) / (ms_sample * 1e-3) / 1e9, 1),
                   "what": "vt_draft_sample: one multinomial draw per row (Gumbel-max), cold"},
        "untrimmed": {"V_high": w.V, "us_per_call": round(us_untrim, 3),
                      "trim_speedup": round(us_untrim / (ms_step * 1000), 3)},
        "prep": {"count_us": round(us_count, 2),
                 "count_GB_per_s": round(prep_bytes_count / (us_count * 1e-6) / 1e9, 1),
                 "select_us": round(us_select, 2),
                 "gather_us": round(us_gather, 2),
                 "gather_GB_per_s": round(prep_bytes_gather / (us_gather * 1e-6) / 1e9, 1),
                 "coverage": round(cov, 6),
                 "coverage_curve_us": round(us_cov, 2),
                 "v_high_for_90pct": v_high_90},
        "pipeline_us": round(us_pipe, 2),
    }
    if M > 2:
        # The wide-tree path is a dense bf16 contraction on the matrix cores: report its
        # rate against the dense bf16 peak. M is padded to whole 16-row MFMA tiles.
        fl = 2.0 * M * V_high * d
        fl_issued = 2.0 * (-(-M // 16) * 16) * V_high * d
        out["mfma"] = {"useful_TFLOP_per_s": round(fl / (ms_step * 1e-3) / 1e12, 1),
                       "issued_TFLOP_per_s": round(fl_issued / (ms_step * 1e-3) / 1e12, 1),
                       "peak_TFLOP_per_s": MFMA_BF16_PEAK_TFLOPS,
                       "frac": round(fl / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                       "flops_per_byte": round(fl / nb, 2),
                       "ridge_flops_per_byte": round(MFMA_BF16_PEAK_TFLOPS / (HBM_PEAK_GBS / 1000), 1),
                       "over": "the whole call (pack + contraction + merge)"}
    if sweep is not None:
        out["sweep"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
