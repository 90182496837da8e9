#!/usr/bin/env python3
"""Throughput of the LightningIndexer hot path on one MI355X.

One step = one full pass of the hot path (score kernel + top-k kernel, i.e.
li_score then li_topk through the C ABI) over one batch of seeded synthetic
input already resident in HBM. The default workload is the 8K causal prefill
(B=1, S1=S2=8192, N1=64, N2=1, D=128, bf16 q/k, bf16 weights, k=2048,
right-down causal, BSND); the other seeded workloads can be selected with
--workload.

Prints ONE JSON line. `value` is indexed query tokens per second; the line
also carries the score kernel's TFLOP/s against the MFMA peak (or its GB/s
against HBM when the workload is bandwidth-bound), the top-k kernel's GB/s,
a `roofline` object for the dominant kernel and a `cpu_baseline` object: the
plain C++ fp64 CPU oracle (one thread per available core) timed on a bounded
random sample of the same rows on this host.

Timing: after W eager warmup steps, K steps (li_score + li_topk each) are
captured as one HIP graph, replayed once untimed and once between two HIP
events on the stream it runs on (ms_per_step = elapsed / K); K launches of the
score kernel alone and of the top-k alone are timed the same way (score_ms,
topk_ms, and the roofline's achieved rate). --eager times K eagerly launched
steps instead. The defaults (200 warmup steps, 200 timed steps: about 0.2 s of
GPU work on the headline workload) time the kernels at the clocks they settle
to under load; a few steps after a cold start read 2-3% slower.

Cold timings (`cold` in the JSON line): each kernel is also launched
--cold-reps times right after a 512 MiB fill kernel that evicts the Infinity
Cache and every L2, HIP events on the launch stream around the kernel alone;
the median is reported with the HBM fraction it implies. `launch_stats` gives
the median, p10 and p90 of per-launch times, warm (--launch-reps launches of
each kernel back to back, each between its own HIP events) and cold (the
launches above). `measured_peaks`
gives this box's own device-copy rate and hipBLASLt bf16 and fp8 GEMM rates
(torch library calls, context for the spec peaks only).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexed query tokens/s + score TFLOP/s (% MFMA peak), S=8K causal prefill"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "e4m3fn": 5000.0, "i8": 5000.0}
PEAK_HBM_GBS = 8000.0
SCORE_SOURCES = ("sparse_attention_top_amd/csrc/li_score.hip",
                 "sparse_attention_top_amd/csrc/li_internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_score_bytes(wl, pairs):
    """Bytes the score kernel must move at least once: Q, W, scales, each key of
    each sequence once, and one float32 per visible pair written (pairs = the
    visible (query row, key) count of the library's task table)."""
    es = 1 if wl.qk_dtype in ("e4m3fn", "i8") else 2
    ws = 4 if wl.w_dtype == "f32" else 2
    rows = int(sum(int(x) for x in wl.seqlens_q))
    keys = int(sum(int(x) for x in wl.seqlens_k))
    b = rows * wl.N1 * (wl.D * es + ws) + keys * wl.N2 * wl.D * es
    if wl.quant:
        b += rows * wl.N1 * 4 + keys * wl.N2 * 4
    return b + 4 * int(pairs)


def host_threads():
    """Threads the CPU baseline may use: the process's CPU share (affinity, and
    OMP_NUM_THREADS where the host sets it)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(omp))) if omp.isdigit() and int(omp) > 0 else max(1, n)


def cpu_baseline(wl, seconds, seed=1234):
    """The plain C++17 fp64 oracle (one std::thread per core) on a random sample
    of the workload's rows, for about `seconds` of wall time."""
    import numpy as np

    from oracle import liref
    rows = [(b, i) for b in range(wl.B) for i in range(int(wl.seqlens_q[b]))]
    order = np.random.default_rng(seed).permutation(len(rows))
    threads = host_threads()
    chunk = 4 * threads
    done, used, t0 = 0, threads, time.perf_counter()
    while done < len(rows) and time.perf_counter() - t0 < seconds:
        sel = [rows[j] for j in order[done:done + chunk]]
        _, _, used = liref.run(wl, rows=sel, nthreads=threads)
        done += len(sel)
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{done} query rows drawn uniformly at random (seed {seed}) from the "
                      f"{len(rows)} rows of the same workload, {el:.1f} s of the C++ fp64 "
                      f"oracle on {used} threads (host: {os.cpu_count()} CPUs, "
                      f"{host_threads()} available)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="dsa_prefill")
    ap.add_argument("--return-value", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch every step eagerly instead of replaying captured graphs")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="launches of each kernel timed after a 512 MiB cache flush (0: none)")
    ap.add_argument("--launch-reps", type=int, default=50,
                    help="warm launches of each kernel timed one by one (median, p10, p90; 0: none)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the on-box reference rates (device copy, bf16 GEMM)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the indexer on one GPU only: rows shard across GPUs with "
              "no exchange, so the multi-GPU figure is N times the one-GPU rate and is not "
              "run here.", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_top_amd import binding as B
    from sparse_attention_top_amd import indexer as I
    from sparse_attention_top_amd import synth

    if args.workload not in synth.CONFIGS:
        sys.exit(f"unknown workload {args.workload}; choose from {list(synth.CONFIGS)}")
    t_gen = time.perf_counter()
    wl = synth.CONFIGS[args.workload]()
    print(f"[bench] generated {args.workload} in {time.perf_counter() - t_gen:.1f}s", flush=True,
          file=sys.stderr)
    dev = "cuda"
    dw = I.upload(wl, dev, return_value=args.return_value)
    plan = I.make_plan(dw.problem, dw.lengths, dev)
    p = dw.problem
    shape = I.output_shape(p)
    idx = torch.empty(shape, dtype=torch.int32, device=dev)
    val = torch.empty(shape if p.return_value else (0,), dtype=torch.float32, device=dev)
    inp = dw.inputs()
    stream = torch.cuda.current_stream()
    mh, md, ws, wsb = plan.meta_host, int(plan.meta_dev.data_ptr()), int(plan.ws.data_ptr()), \
        plan.ws_bytes
    ip, vp = int(idx.data_ptr()), (int(val.data_ptr()) if p.return_value else 0)

    def cur():
        return int(torch.cuda.current_stream().cuda_stream)

    def score():
        B.li_score(p, inp, mh, md, ws, wsb, cur())

    def topk():
        B.li_topk(p, mh, md, ws, wsb, ip, vp, cur())

    def step():
        score()
        topk()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", flush=True, file=sys.stderr)

    K = args.steps
    timing = "eager" if args.eager else "graph"
    if not args.eager:
        # K steps (and K launches of each kernel alone) captured as one HIP
        # graph each and replayed once between two HIP events on the stream
        # it runs on: the timed region then holds GPU work only (eager
        # launches through ctypes leave host gaps that short workloads feel).
        try:
            graphs = {}
            for name, fn in (("step", step), ("score", score), ("topk", topk)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(K):
                        fn()
                graphs[name] = g
            torch.cuda.synchronize()
        except RuntimeError as e:   # capture unavailable: time eager launches instead
            print(f"[bench] graph capture failed ({e}); timing eager launches", flush=True,
                  file=sys.stderr)
            timing = "eager"
            torch.cuda.synchronize()
    if timing == "eager":
        # Launch by launch, HIP events between the kernels of every step.
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for s in range(K):
            ev[s][0].record(stream)
            score()
            ev[s][1].record(stream)
            topk()
            ev[s][2].record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(end) / K
        score_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
        topk_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    else:
        def timed(g):
            g.replay()   # one untimed replay (graph upload)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / K

        ms_per_step = timed(graphs["step"])
        score_ms = timed(graphs["score"])
        topk_ms = timed(graphs["topk"])
        del graphs
    print(f"[bench] timed {K} steps: {ms_per_step:.3f} ms/step (score {score_ms:.3f}, "
          f"top-k {topk_ms:.3f})", flush=True, file=sys.stderr)

    # Per-launch distributions (median, p10, p90): each launch
    # bracketed by its own HIP events on the launch stream, warm (back to back
    # after the graphs) and cold (below).
    def launch_times(fn, reps, flush=None):
        ts = []
        for r in range(reps):
            if flush is not None:
                flush.fill_(float(r))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return ts

    def quantiles(ts):
        v = sorted(ts)
        q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
        return {"median": round(q(0.5), 4), "p10": round(q(0.1), 4), "p90": round(q(0.9), 4)}

    warm = None
    if args.launch_reps > 0:
        warm = {"score": launch_times(score, args.launch_reps), "topk": launch_times(topk, args.launch_reps)}

    # Cold timings: each launch follows a 512 MiB fill kernel (twice the 256 MB
    # Infinity Cache plus every L2), so its inputs come from HBM; HIP events on
    # the launch stream bracket the kernel alone. Median over the launches.
    cold = None
    if args.cold_reps > 0:
        flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)

        cold = {"score": launch_times(score, args.cold_reps, flush),
                "topk": launch_times(topk, args.cold_reps, flush)}
        cold["score_ms"] = quantiles(cold["score"])["median"]
        cold["topk_ms"] = quantiles(cold["topk"])["median"]
        del flush
        print(f"[bench] cold (after a 512 MiB flush): score {cold['score_ms']:.3f} ms, "
              f"top-k {cold['topk_ms']:.3f} ms", flush=True, file=sys.stderr)

    # On-box reference rates next to the spec peaks: a 1 GiB device copy and a
    # bf16 8192^3 GEMM (torch library calls; context only, not the indexer).
    peaks = None
    if not args.no_peaks:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        m = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        n = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)

        def rate(fn, reps):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps * 1e-3

        t_copy = rate(lambda: b.copy_(a), 10)
        t_gemm = rate(lambda: torch.matmul(m, n), 10)
        peaks = {"device_copy_gbs": round(2 * a.numel() * 4 / t_copy / 1e9, 1),
                 "bf16_gemm_tflops": round(2 * 8192 ** 3 / t_gemm / 1e12, 1)}
        # fp8 (e4m3fn) GEMM through torch's scaled matmul, the same shape; null
        # where this torch build has no such path.
        try:
            m8 = m.to(torch.float8_e4m3fn)
            n8 = n.t().contiguous().to(torch.float8_e4m3fn).t()   # column-major right operand
            one = torch.ones((), device=dev, dtype=torch.float32)
            t_f8 = rate(lambda: torch._scaled_mm(m8, n8, scale_a=one, scale_b=one,
                                                 out_dtype=torch.bfloat16), 10)
            peaks["fp8_gemm_tflops"] = round(2 * 8192 ** 3 / t_f8 / 1e12, 1)
            del m8, n8
        except (RuntimeError, AttributeError, TypeError) as e:
            print(f"[bench] fp8 GEMM rate unavailable ({e})", flush=True, file=sys.stderr)
            peaks["fp8_gemm_tflops"] = None
        del a, b, m, n

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: 3 x 1 GiB device copy done", flush=True,
              file=sys.stderr)

    rows = wl.num_rows
    pairs = int(plan.header["visible_pairs"])
    flops = 2.0 * wl.N1 * wl.D * pairs
    score_tflops = flops / (score_ms * 1e-3) / 1e12
    sbytes = algorithmic_score_bytes(wl, pairs)
    score_gbs = sbytes / (score_ms * 1e-3) / 1e9
    kk = wl.sparse_count
    tbytes = 4 * pairs + rows * wl.N2 * kk * (8 if p.return_value else 4)
    topk_gbs = tbytes / (topk_ms * 1e-3) / 1e9
    peak_mfma = PEAK_MFMA_TFLOPS[wl.qk_dtype]
    ridge = peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm_bound = flops / sbytes < ridge

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_digest") == source_digest(SCORE_SOURCES) and \
                tr.get("workload") == args.workload:
            traffic = tr.get("bytes_per_launch")
    if hbm_bound:
        roof = {"kernel": "score_kernel", "bound": "hbm", "achieved": round(score_gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(score_gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": sbytes}
    else:
        roof = {"kernel": "score_kernel", "bound": "mfma", "achieved": round(score_tflops, 1),
                "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": round(score_tflops / peak_mfma, 4), "traffic": traffic,
                "algorithmic_flops": flops}

    out = {
        "metric": METRIC,
        "value": round(rows / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.qk_dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": wl.B, "S1": wl.S1, "S2": wl.S2, "N1": wl.N1,
                   "N2": wl.N2, "D": wl.D, "layout_q": wl.layout_q, "layout_k": wl.layout_k,
                   "sparse_count": kk, "sparse_mode": wl.sparse_mode,
                   "return_value": bool(p.return_value), "query_rows": rows,
                   "visible_pairs": pairs, "parallelism": "single GPU", "timing": timing},
        "score_tflops": round(score_tflops, 1),
        "score_frac_mfma_peak": round(score_tflops / peak_mfma, 4),
        "score_ms": round(score_ms, 4),
        "topk_ms": round(topk_ms, 4),
        "topk_gbs": round(topk_gbs, 1),
        "topk_frac_hbm_peak": round(topk_gbs / PEAK_HBM_GBS, 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if cold is not None:
        out["cold"] = {"score_ms": round(cold["score_ms"], 4), "topk_ms": round(cold["topk_ms"], 4),
                       "score_tflops": round(flops / (cold["score_ms"] * 1e-3) / 1e12, 1),
                       "topk_gbs": round(tbytes / (cold["topk_ms"] * 1e-3) / 1e9, 1),
                       "topk_frac_hbm_peak": round(tbytes / (cold["topk_ms"] * 1e-3) / 1e9 /
                                                   PEAK_HBM_GBS, 4),
                       "flush_bytes": 1 << 29, "launches": args.cold_reps, "timing": "eager, median"}
    if warm is not None or cold is not None:
        ls = {"timing": "eager, HIP events around each launch"}
        if warm is not None:
            ls["warm"] = {"launches": args.launch_reps, "score_ms": quantiles(warm["score"]),
                          "topk_ms": quantiles(warm["topk"])}
        if cold is not None:
            ls["cold"] = {"launches": args.cold_reps, "score_ms": quantiles(cold["score"]),
                          "topk_ms": quantiles(cold["topk"])}
        out["launch_stats"] = ls
    if peaks is not None:
        out["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", flush=True, file=sys.stderr)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
