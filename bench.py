#!/usr/bin/env python3
"""Benchmark of the fused projection -> residual add -> RMSNorm call on one MI355X.

A step is one fused call over one batch of T tokens of a workload (all steps of the path:
the projection of every row block, the hand-off of its result, the residual add and the
RMSNorm), with inputs already resident in HBM.  The default workload is the Llama-3-8B-shaped
o_proj prefill (T=2048, K=H=4096, bf16, standard RMSNorm).  The fused forms are the
microchunk pipeline at each of the workload's chunk sizes ({256, 512} for o_proj) and the
single launch; the fastest is the headline.  The conventional path is timed beside them.
Prints one JSON line.

    python bench.py [--steps 50] [--warmup 10] [--workload o_proj] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="o_proj")
    ap.add_argument("--microchunk", type=int, default=0, help="0: every chunk size of the workload")
    ap.add_argument("--only-single", action="store_true",
                    help="time only the single-launch fused form (profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip the load-time tuning (chunk projections use the time model)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-dir", default=os.path.join(ROOT, "profiles"),
                    help="directory of traffic_*.json counter summaries (measured HBM bytes per "
                         "launch of the headline kernel)")
    ap.add_argument("--tune-sweep", action="store_true",
                    help="run the token-threshold search on the K=H=8192 sweep and print it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--addnorm-roofline", action="store_true",
                    help="HBM rate of the conventional path's add/norm kernel on every workload, "
                         "Infinity Cache warm and flushed, beside a plain device copy")
    ap.add_argument("--silu-mul", action="store_true",
                    help="HBM rate of the SiluAndMul kernel (down_proj and Gemma intermediate "
                         "sizes, warm and flushed) and the down_proj block it opens")
    ap.add_argument("--cu-split", default="",
                    help="comma-separated CU counts reserved for the add/norm stream (0 = the "
                         "ping-pong schedule): time the pipeline of the workload at each chunk "
                         "size and split, round-robin, and print the table")
    ap.add_argument("--phases", default="",
                    help="comma-separated workloads: in-kernel phase and clock stamps of the single "
                         "launch, from the diagnostic library libprojaddnorm_stamps.so (same "
                         "kernels with stamps); writes the summary to --phases-out")
    ap.add_argument("--phases-out", default="", help="markdown summary of --phases (else stdout)")
    ap.add_argument("--tp-share", default="",
                    help="comma-separated tensor-parallel degrees P: time one rank's share of "
                         "the workload (projection over K/P, add/norm of T/P rows with P fp32 "
                         "partials) and print the table")
    return ap.parse_args()


def time_steps(call, steps: int, warmup: int, torch):
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def evict(flush) -> None:
    """Evicts the call's operands from the caches by READING a buffer twice the size of the
    256 MB Infinity Cache.  A write of that buffer would evict them too, but would leave the
    cache full of dirty lines whose write-back the next kernel's misses then pay for (a plain
    50 MiB copy measured 33 us after such a write and 18 us after this read)."""
    flush.sum()


def per_call_stats(call, r, r0, steps: int, torch, stream, flush=None) -> dict:
    """Single calls timed with events on the calling stream.  Before each call (untimed) the
    residual is restored from a pristine copy and, with `flush`, the caches are evicted, so that
    none of the call's operands is cached."""
    times = []
    for i in range(steps + 3):
        r.copy_(r0)
        if flush is not None:
            evict(flush)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        if i >= 3:
            times.append(e0.elapsed_time(e1))
    t = np.array(times)
    return {"median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90)), "calls": len(times)}


def add_per_call_stats(result, fused_call, conventional, r, steps, torch, stream, dev,
                       form: str) -> None:
    r0 = r.clone()
    flush = torch.zeros(1 << 27, dtype=torch.float32, device=dev)  # 512 MB
    result["per_call"] = {
        "form": form,
        "fused_warm": per_call_stats(fused_call, r, r0, steps, torch, stream),
        "fused_flushed": per_call_stats(fused_call, r, r0, steps, torch, stream, flush),
        "conventional_warm": per_call_stats(conventional, r, r0, steps, torch, stream),
        "conventional_flushed": per_call_stats(conventional, r, r0, steps, torch, stream, flush)}
    del flush, r0
    pc = result["per_call"]
    log(f"per call (median ms, warm / flushed): fused {pc['fused_warm']['median_ms']:.4f} / "
        f"{pc['fused_flushed']['median_ms']:.4f}, conventional "
        f"{pc['conventional_warm']['median_ms']:.4f} / "
        f"{pc['conventional_flushed']['median_ms']:.4f}")


def traffic_label(workload: str, mc, chunk_cfgs: dict) -> str:
    """Label of a traffic measurement: workload, fused form (chunk size or "single") and the
    projection configuration it ran with (counters taken under another configuration do not
    apply)."""
    key = "mc=single" if mc == "single" else f"mc={mc}"
    return f"{workload}:{key}:{chunk_cfgs.get(str(mc), 'model')}"


def cpu_baseline(d, seconds: float) -> dict:
    """The oracle, as it stands, on a bounded sample of the workload's tokens."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    rows = min(d["T"], 256)
    x, r = d["x"][:rows], d["residual"][:rows]
    reps, t_total = 0, 0.0
    while t_total < seconds and reps < 1000:
        t0 = time.perf_counter()
        oracle.proj_add_rmsnorm(x, d["W"], r, d["norm_w"], d["eps"], d["norm_kind"], "fused")
        t_total += time.perf_counter() - t0
        reps += 1
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                       None)
    except OSError:  # pragma: no cover
        pass
    return {"value": rows * reps / t_total, "unit": "tokens/s", "cores": int(threads),
            "cpu": cpu, "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"first {rows} of {d['T']} tokens, {reps} calls of the float64 oracle "
                      f"({t_total:.1f} s); rows are independent, so tokens/s scales to the "
                      f"full batch"}


def under_profiler() -> bool:
    """True when this process runs under rocprofv3 (its tool library is preloaded)."""
    return ("rocprof" in os.environ.get("LD_PRELOAD", "")
            or any(k.startswith(("ROCPROF_", "ROCPROFILER_")) for k in os.environ))


def clock_settings() -> dict:
    """The GPU's clock settings as amd-smi reports them (run as a child process before this
    process initialises the GPU): per-XCD shader-clock range, whether it is locked, and the
    memory clock.  Clocks are left at their defaults; None when amd-smi is unavailable."""
    import shutil
    import subprocess
    if under_profiler():
        # A profiler's preloaded library reaches the child too and opens the GPU there before
        # amd-smi's interpreter line replaces the process, which must not happen.
        return None
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    try:
        proc = subprocess.run([exe, "metric", "--clock", "--json"], capture_output=True,
                              text=True, timeout=60)
        gpu = json.loads(proc.stdout)["gpu_data"][0]["clock"]
    except Exception:  # pragma: no cover - depends on the box
        return None

    def mhz(v):
        return v["value"] if isinstance(v, dict) else None
    gfx = [v for k, v in gpu.items() if k.startswith("gfx_")]
    mem = gpu.get("mem_0", {})
    return {"source": "amd-smi metric --clock",
            "sclk_max_MHz": sorted({mhz(v.get("max_clk")) for v in gfx} - {None}),
            "sclk_min_MHz": sorted({mhz(v.get("min_clk")) for v in gfx} - {None}),
            "sclk_locked": sorted({v.get("clk_locked") for v in gfx}),
            "xcds": len(gfx), "mclk_MHz": mhz(mem.get("clk"))}


def threshold_sweep(pr, args) -> dict:
    """Token-threshold search over the long-prefill sweep (K = H = 8192, T in the sweep grid):
    the library's tuner checks every fused candidate (each chunk size and the single launch)
    against the conventional path on its own uniform synthetic data, times all of them
    round-robin, and derives the crossover token count.  Times are the tuner's medians."""
    import synth
    grid = list(synth.SWEEP_T)
    mcs = [512, 1024, 2048]
    t0 = time.perf_counter()
    rep = pr.pr_tune([8192], [8192], pr.PR_NORM_STANDARD, grid, mcs, reps=max(args.steps // 5, 5))
    rows = []
    for i, T in enumerate(grid):
        t = rep["timings"][0][i]
        rows.append({"T": T, "conventional_ms": t[0] * 1e3,
                     "best_fused_ms": t[1] * 1e3 if t[1] > 0 else None,
                     "fused_ms": {str(m): (t[2 + j] * 1e3 if t[2 + j] > 0 else None)
                                  for j, m in enumerate(mcs)},
                     "single_launch_ms": t[2 + len(mcs)] * 1e3 if t[2 + len(mcs)] > 0 else None})
    thr = rep["threshold_tokens"]
    res = {"K": 8192, "H": 8192, "T_grid": grid, "microchunks": mcs, "rows": rows,
           "n_checked": rep["n_checked"], "n_rejected": rep["n_rejected"],
           "threshold_tokens": None if thr == pr.INT32_MAX else thr,
           "seconds": time.perf_counter() - t0}
    log(f"threshold sweep (K=H=8192): crossover T = {res['threshold_tokens']} "
        f"({res['n_checked']} candidates checked, {res['n_rejected']} rejected, "
        f"{res['seconds']:.1f} s)")
    return res


def tune_sweep(pr, torch, args) -> int:
    """The threshold sweep alone: prints its table as one JSON line."""
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    print(json.dumps({"tune_sweep": threshold_sweep(pr, args)}), flush=True)
    return 0


def addnorm_roofline(pr, torch, args) -> int:
    """The add/norm kernel alone, as the conventional path launches it after the projection:
    algorithmic bytes per element (y read: 2 for bf16, 4 per fp32 plane; r read 4, r write 4,
    out write 2) over its event-timed duration, with the Infinity Cache warm, flushed (a 512 MB
    read before each call) and dirty (a 512 MB write before each call, whose write-backs the call
    then shares the memory with), against 8 TB/s and against a device copy of the same bytes
    (half read, half written) after the same read flush."""
    import synth
    dev = "cuda:0"
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    flush = torch.zeros(1 << 27, dtype=torch.float32, device=dev)
    names = ["o_proj", "down_proj", "gemma", "sweep_T8192"]
    rows = []
    for name in names:
        wl = synth.WORKLOADS[name]
        T, K, H = wl.T, wl.K, wl.H
        d = synth.make_inputs(wl, seed=0)
        x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
        W_src = torch.from_numpy(d["W"].view(np.int16)).to(dev)
        Wp = torch.empty(K * H, dtype=torch.int16, device=dev)
        pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
        del W_src
        r = torch.from_numpy(d["residual"]).to(dev)
        r0 = r.clone()
        w = torch.from_numpy(d["norm_w"]).to(dev)
        out = torch.empty((T, H), dtype=torch.int16, device=dev)
        split = pr.pr_select(T, K, H, pr.PR_SELECT_UNFUSED)["split_k"]
        per_elem = (2 if split == 1 else 4 * split) + 10
        nbytes = per_elem * T * H
        res = {"workload": name, "T": T, "H": H, "y": "bf16" if split == 1 else f"{split} fp32 planes",
               "bytes_per_elem": per_elem, "bytes": nbytes}
        for mode in ("warm", "flushed", "dirty"):
            ts = []
            for i in range(max(args.steps // 5, 5) + 2):
                r.copy_(r0)
                if mode == "flushed":
                    evict(flush)
                elif mode == "dirty":
                    flush.fill_(float(i))
                pr.pr_profile_enable(True)
                pr.proj_add_rmsnorm_unfused(x, Wp, r, w, d["eps"], T, K, H, wl.norm_kind, out)
                prof = pr.pr_profile_read()
                pr.pr_profile_enable(False)
                if i >= 2:
                    ts.append(prof["addnorm_ms"] / max(prof["addnorm_launches"], 1))
            t = float(np.median(ts)) / 1e3
            res[f"{mode}_us"] = t * 1e6
            res[f"{mode}_GBs"] = nbytes / t / 1e9
        # a device copy of the same bytes: half read, half written
        src = torch.empty(nbytes // 2 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        cts = []
        for i in range(7):
            evict(flush)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            e1.synchronize()
            if i >= 2:
                cts.append(e0.elapsed_time(e1) / 1e3)
        res["copy_flushed_GBs"] = nbytes / float(np.median(cts)) / 1e9
        res["frac_hbm_peak_flushed"] = res["flushed_GBs"] / PEAK_HBM_GBS
        rows.append(res)
        log(f"{name}: add/norm {res['warm_us']:.1f} us warm ({res['warm_GBs']:.0f} GB/s), "
            f"{res['flushed_us']:.1f} us flushed ({res['flushed_GBs']:.0f} GB/s), "
            f"{res['dirty_us']:.1f} us dirty ({res['dirty_GBs']:.0f} GB/s); copy of the same "
            f"bytes {res['copy_flushed_GBs']:.0f} GB/s flushed")
        del x, Wp, r, r0, w, out, src, dst
        torch.cuda.empty_cache()
    print(json.dumps({"addnorm_roofline": rows, "peak_GBs": PEAK_HBM_GBS}), flush=True)
    return 0


def silu_mul_roofline(pr, torch, args) -> int:
    """SiluAndMul from the merged gate/up output: algorithmic bytes per element of x (gate 2 +
    up 2 read, x 2 written) over the event-timed kernel, warm and flushed (a 512 MB read before
    each call), against 8 TB/s; then the down_proj block (SiluAndMul followed by the single
    launch), the same block in one launch with SiluAndMul in the main loop, and the single
    launch alone, back to back, the three series alternated five times (medians)."""
    import synth
    dev = "cuda:0"
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    flush = torch.zeros(1 << 27, dtype=torch.float32, device=dev)
    rows = []
    for name in ("down_proj", "gemma"):
        wl = synth.WORKLOADS[name]
        T, K, H = wl.T, wl.K, wl.H
        d = synth.gate_up_inputs(T, K, H, seed=0, K_real=wl.K_real, eps=wl.eps)
        gu = torch.from_numpy(d["gate_up"].view(np.int16)).to(dev)
        x = torch.empty((T, K), dtype=torch.int16, device=dev)
        nbytes = 6 * T * K
        res = {"workload": name, "T": T, "K": K, "bytes": nbytes}
        for mode in ("warm", "flushed"):
            ts = []
            for i in range(max(args.steps // 2, 10) + 2):
                if mode == "flushed":
                    evict(flush)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                pr.pr_silu_mul(gu, x, T, K, stream)
                e1.record(stream)
                e1.synchronize()
                if i >= 2:
                    ts.append(e0.elapsed_time(e1) / 1e3)
            t = float(np.median(ts))
            res[f"{mode}_us"] = t * 1e6
            res[f"{mode}_GBs"] = nbytes / t / 1e9
        res["frac_hbm_peak_flushed"] = res["flushed_GBs"] / PEAK_HBM_GBS
        # the block: SiluAndMul then the single launch, against the single launch alone
        W_src = torch.from_numpy(d["W"].view(np.int16)).to(dev)
        Wp = torch.empty(K * H, dtype=torch.int16, device=dev)
        pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
        del W_src
        r = torch.from_numpy(d["residual"]).to(dev)
        w = torch.from_numpy(d["norm_w"]).to(dev)
        out = torch.empty((T, H), dtype=torch.int16, device=dev)

        def single():
            pr.proj_add_rmsnorm_single_launch(x, Wp, r, w, d["eps"], T, K, H, wl.norm_kind, out,
                                              stream)

        def block():
            pr.pr_silu_mul(gu, x, T, K, stream)
            single()

        def fused_block():
            pr.proj_add_rmsnorm_silu(gu, Wp, r, w, d["eps"], T, K, H, wl.norm_kind, out, stream)
        # alternated, so that clock drift between the series cancels
        series = {"single_launch": [], "block": [], "fused_block": []}
        for _ in range(5):
            for label, fn in (("single_launch", single), ("block", block),
                              ("fused_block", fused_block)):
                el = time_steps(fn, args.steps, args.warmup, torch)
                series[label].append(el * 1e3 / args.steps)
        for label, v in series.items():
            res[f"{label}_ms"] = float(np.median(v))
        if pr.pr_device_status(stream) != 0:
            raise SystemExit("single-launch status bits set: a row wait gave up")
        rows.append(res)
        log(f"{name}: silu_mul {res['warm_us']:.1f} us warm ({res['warm_GBs']:.0f} GB/s), "
            f"{res['flushed_us']:.1f} us flushed ({res['flushed_GBs']:.0f} GB/s); block "
            f"{res['block_ms']:.4f} ms (SiluAndMul in the main loop: "
            f"{res['fused_block_ms']:.4f} ms) vs single launch {res['single_launch_ms']:.4f} ms")
        del gu, x, Wp, r, w, out
        torch.cuda.empty_cache()
    print(json.dumps({"silu_mul": rows, "peak_GBs": PEAK_HBM_GBS}), flush=True)
    return 0


def conventional_addnorm_flushed(pr, torch, x, Wp, r, w, out, d, wl, steps, stream) -> dict:
    """The conventional path's add/norm kernel (the pass after the projection) with no operand
    in the caches: before each call the residual is restored and a 512 MB buffer is read.  Its
    algorithmic bytes per element are y read (2 for bf16 y, 4 per fp32 plane), r read 4, r write
    4, out write 2; the rate is those bytes over the kernel's event-timed duration."""
    T, K, H = d["T"], d["K"], d["H"]
    flush = torch.zeros(1 << 27, dtype=torch.float32, device=r.device)
    r0 = r.clone()
    split = pr.pr_select(T, K, H, pr.PR_SELECT_UNFUSED)["split_k"]
    per_elem = (2 if split == 1 else 4 * split) + 10
    ts = []
    for i in range(max(steps // 2, 8) + 2):
        r.copy_(r0)
        evict(flush)
        pr.pr_profile_enable(True)
        pr.proj_add_rmsnorm_unfused(x, Wp, r, w, d["eps"], T, K, H, wl.norm_kind, out, stream)
        prof = pr.pr_profile_read()
        pr.pr_profile_enable(False)
        if i >= 2:
            ts.append(prof["addnorm_ms"] / max(prof["addnorm_launches"], 1) / 1e3)
    r.copy_(r0)
    del flush, r0
    t = float(np.median(ts))
    gbs = per_elem * T * H / t / 1e9
    log(f"conventional add/norm, flushed: {t * 1e6:.1f} us, {gbs:.0f} GB/s "
        f"({gbs / PEAK_HBM_GBS:.3f} of 8 TB/s)")
    return {"kernel": "add_rmsnorm_kernel", "cache": "flushed (512 MB read before each call)",
            "y": "bf16" if split == 1 else f"{split} fp32 planes", "bytes_per_elem": per_elem,
            "median_us": t * 1e6, "GBs": gbs, "peak_GBs": PEAK_HBM_GBS,
            "frac": gbs / PEAK_HBM_GBS, "calls": len(ts)}


def fp8_entry(pr, torch, x, W_src, r, w, out, d, norm_kind, scale_rows, args, stream) -> dict:
    """The same region with the FP8 (OCP E4M3) projection.  Load time (untimed): the weight is
    quantised with one per-tensor scale and laid out for the matrix cores.  A step: the
    activations quantised with one scale per `scale_rows` tokens, then the FP8 single launch.
    The kernel's own duration comes from the library's events; its rate is priced against the
    dense fp8 peak."""
    T, K, H = d["T"], d["K"], d["H"]
    dev = r.device
    wq = torch.empty((H, K), dtype=torch.uint8, device=dev)
    sw = torch.empty(1, dtype=torch.float32, device=dev)
    pr.pr_quantize_fp8(W_src, wq, sw, H, K, H, stream)
    Wp8 = torch.empty(K * H, dtype=torch.uint8, device=dev)
    pr.pr_prepare_weight_fp8(wq, pr.PR_WEIGHT_OUT_IN, Wp8, K, H, stream)
    xq = torch.empty((T, K), dtype=torch.uint8, device=dev)
    sx = torch.empty(((T - 1) // scale_rows + 1,), dtype=torch.float32, device=dev)

    def step():
        pr.pr_quantize_fp8(x, xq, sx, T, K, scale_rows, stream)
        pr.proj_add_rmsnorm_fp8(xq, sx, scale_rows, Wp8, sw, r, w, d["eps"], T, K, H, norm_kind,
                                out, stream)

    steps = max(args.steps, 5)
    el = time_steps(step, steps, max(args.warmup, 2), torch)
    pr.pr_profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = pr.pr_profile_read()
    pr.pr_profile_enable(False)
    if pr.pr_device_status(stream) != 0:
        raise SystemExit("FP8 single-launch status bits set: a row wait gave up")
    flops = 2.0 * T * K * H
    k_s = prof["gemm_ms"] / max(prof["gemm_launches"], 1) / 1e3
    res = {"format": "OCP E4M3 (x per-group and W per-tensor fp32 scales)",
           "scale_rows": scale_rows, "ms_per_step": el * 1e3 / steps,
           "tokens_per_s": T * steps / el, "step_tflops": flops * steps / el / 1e12,
           "kernel": "gemm_add_rmsnorm_kernel (FP8)", "kernel_avg_us": k_s * 1e6,
           "kernel_tflops": flops / k_s / 1e12, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
           "frac": flops / k_s / 1e12 / PEAK_FP8_TFLOPS,
           "quantize_us_per_step": max(el / steps - k_s, 0.0) * 1e6}
    log(f"fp8: {res['ms_per_step']:.4f} ms/step (quantise + single launch), kernel "
        f"{res['kernel_avg_us']:.1f} us = {res['kernel_tflops']:.0f} TFLOP/s, "
        f"{res['frac']:.3f} of the fp8 peak")
    if scale_rows != 1:
        # The same step with per-token activation scales (rows of up to 8192 columns are
        # quantised in one pass).
        sx1 = torch.empty((T,), dtype=torch.float32, device=dev)

        def step1():
            pr.pr_quantize_fp8(x, xq, sx1, T, K, 1, stream)
            pr.proj_add_rmsnorm_fp8(xq, sx1, 1, Wp8, sw, r, w, d["eps"], T, K, H, norm_kind, out,
                                    stream)

        el1 = time_steps(step1, steps, max(args.warmup, 2), torch)
        if pr.pr_device_status(stream) != 0:
            raise SystemExit("FP8 single-launch status bits set: a row wait gave up")
        res["per_token"] = {"scale_rows": 1, "ms_per_step": el1 * 1e3 / steps,
                            "tokens_per_s": T * steps / el1,
                            "step_tflops": flops * steps / el1 / 1e12}
        log(f"fp8, per-token scales: {res['per_token']['ms_per_step']:.4f} ms/step")
        del sx1
    del wq, sw, Wp8, xq, sx
    return res


def down_proj_entry(pr, torch, args, stream) -> dict:
    """The second 4096-class prefill shape, down_proj (T=4096, K=14336, H=4096, x = silu(a)*b):
    the single launch and the conventional path, timed back to back (the two series
    alternated three times, medians), and the single launch's kernel duration from the
    library's events."""
    import synth
    wl = synth.WORKLOADS["down_proj"]
    T, K, H = wl.T, wl.K, wl.H
    dev = "cuda:0"
    d = synth.make_inputs(wl, seed=0)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    W_src = torch.from_numpy(d["W"].view(np.int16)).to(dev)
    Wp = torch.empty(K * H, dtype=torch.int16, device=dev)
    pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
    r = torch.from_numpy(d["residual"]).to(dev)
    w = torch.from_numpy(d["norm_w"]).to(dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    flops = 2.0 * T * K * H
    steps = max(args.steps // 2, 5)
    calls = {
        "single": lambda: pr.proj_add_rmsnorm_single_launch(x, Wp, r, w, d["eps"], T, K, H,
                                                            wl.norm_kind, out, stream),
        "conventional": lambda: pr.proj_add_rmsnorm_unfused(x, Wp, r, w, d["eps"], T, K, H,
                                                            wl.norm_kind, out, stream)}
    series = {k: [] for k in calls}
    for _ in range(3):
        for k, fn in calls.items():
            series[k].append(time_steps(fn, steps, max(args.warmup // 2, 2), torch) / steps)
    pr.pr_profile_enable(True)
    for _ in range(steps):
        calls["single"]()
    torch.cuda.synchronize()
    prof = pr.pr_profile_read()
    pr.pr_profile_enable(False)
    if pr.pr_device_status(stream) != 0:
        raise SystemExit("single-launch status bits set: a row wait gave up")
    t_s, t_c = float(np.median(series["single"])), float(np.median(series["conventional"]))
    k_s = prof["gemm_ms"] / max(prof["gemm_launches"], 1) / 1e3
    c = pr.pr_select(T, K, H, pr.PR_SINGLE_LAUNCH)
    res = {"workload": "down_proj prefill", "T": T, "K": K, "H": H,
           "single_launch_ms": t_s * 1e3, "tokens_per_s": T / t_s,
           "tflops": flops / t_s / 1e12, "frac_bf16_peak": flops / t_s / 1e12 / PEAK_BF16_TFLOPS,
           "kernel_avg_us": k_s * 1e6, "kernel_tflops": flops / k_s / 1e12,
           "kernel_frac": flops / k_s / 1e12 / PEAK_BF16_TFLOPS,
           "tile": f"{c['gemm_bm']}x{c['gemm_bn']} {c['gemm_waves']} waves",
           "conventional_ms": t_c * 1e3, "conventional_tflops": flops / t_c / 1e12}
    res["fp8"] = fp8_entry(pr, torch, x, W_src, r, w, out, d, wl.norm_kind, 512, args, stream)
    del W_src
    log(f"down_proj: single launch {res['single_launch_ms']:.4f} ms ({res['tflops']:.0f} "
        f"TFLOP/s, kernel {res['kernel_avg_us']:.1f} us = {res['kernel_frac']:.3f} of peak), "
        f"conventional {res['conventional_ms']:.4f} ms")
    del x, Wp, r, w, out
    torch.cuda.empty_cache()
    return res


def cu_split_table(pr, torch, args) -> int:
    """The CU-partitioned pipeline against the ping-pong one: for each chunk size of the
    workload and each split (CUs reserved for the add/norm stream; 0 = ping-pong), the call
    time of back-to-back calls.  The splits of one chunk size are timed in rounds, one series
    of `steps` calls each per round, five rounds, medians (clock drift cancels)."""
    import synth
    wl = synth.WORKLOADS[args.workload]
    T, K, H = wl.T, wl.K, wl.H
    dev = "cuda:0"
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    d = synth.make_inputs(wl, seed=0)
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    W_src = torch.from_numpy(d["W"].view(np.int16)).to(dev)
    Wp = torch.empty(K * H, dtype=torch.int16, device=dev)
    pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
    r = torch.from_numpy(d["residual"]).to(dev)
    w = torch.from_numpy(d["norm_w"]).to(dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    splits = [int(v) for v in args.cu_split.split(",") if v != ""]
    if len(splits) > 2 or (len(splits) == 2 and 0 not in splits):
        raise SystemExit("--cu-split takes one split, or 0 and one split: the library keeps one "
                         "CU-masked stream pair per device (run one process per split)")
    rows = []
    conv = lambda: pr.proj_add_rmsnorm_unfused(x, Wp, r, w, d["eps"], T, K, H, wl.norm_kind, out)
    t_conv = float(np.median([time_steps(conv, args.steps, args.warmup, torch) / args.steps
                              for _ in range(3)]))
    for mc in wl.microchunks:
        series = {n: [] for n in splits}
        for _ in range(5):
            for n in splits:
                os.environ["PR_FORCE_CU_SPLIT"] = str(n)
                call = lambda: pr.proj_add_rmsnorm(x, Wp, r, w, d["eps"], T, K, H, mc,
                                                   wl.norm_kind, out)
                series[n].append(time_steps(call, args.steps, args.warmup, torch) / args.steps)
        for n in splits:
            os.environ["PR_FORCE_CU_SPLIT"] = str(n)
            c = pr.pr_select(T, K, H, mc)
            t = float(np.median(series[n]))
            cfg = f"{c['gemm_bm']}x{c['gemm_bn']} split {c['split_k']}"
            rows.append({"mc": mc, "addnorm_cus": n, "ms": t * 1e3, "chunk_projection": cfg})
            log(f"mc={mc} split {n}: {t * 1e3:.4f} ms ({cfg})")
        os.environ.pop("PR_FORCE_CU_SPLIT", None)
    log(f"conventional: {t_conv * 1e3:.4f} ms")
    print(json.dumps({"cu_split": {"workload": wl.name, "T": T, "K": K, "H": H,
                                   "conventional_ms": t_conv * 1e3, "rows": rows}}), flush=True)
    return 0


XGMI_LINK_GBS = 153.0   # one xGMI link, per direction


def tp_share(pr, torch, args) -> int:
    """One rank's share of the row-parallel projection region under tensor parallelism of
    degree P, measured on this GPU: the projection of all T (or one chunk of mc) tokens over the
    rank's K/P input columns into an fp32 partial (pr_project_partial; beside it the library's
    own tile and K split through the fused entry point), and the add/norm of the rank's T/P
    (mc/P) token shard summing P fp32 partials in rank order (pr_add_rmsnorm_partials).  The reduce-scatter of the partials and
    the all-gather of the bf16 output between them are modelled, not run: a one-shot exchange
    in which every rank sends each peer its shard over that peer's own xGMI link."""
    import synth
    wl = synth.WORKLOADS[args.workload]
    T, K, H = wl.T, wl.K, wl.H
    dev = "cuda:0"
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    steps = max(args.steps, 5)

    def per_launch(call, kind):
        for _ in range(max(args.warmup, 2)):
            call()
        torch.cuda.synchronize()
        pr.pr_profile_enable(True)
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        prof = pr.pr_profile_read()
        pr.pr_profile_enable(False)
        ms, n = prof[kind + "_ms"], prof[kind + "_launches"]
        return ms / max(n, 1) * 1e3  # us

    def device_inputs(rows, k):
        d = synth.make_custom(rows, k, H, seed=rows + k, norm_kind=wl.norm_kind, eps=wl.eps,
                              x_dist=wl.x_dist)
        x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
        W_src = torch.from_numpy(d["W"].view(np.int16)).to(dev)
        Wp = torch.empty(k * H, dtype=torch.int16, device=dev)
        pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, k, H)
        r = torch.from_numpy(d["residual"]).to(dev)
        w = torch.from_numpy(d["norm_w"]).to(dev)
        out = torch.empty((rows, H), dtype=torch.int16, device=dev)
        return d, x, Wp, r, w, out

    rows_out = []
    for P in [int(v) for v in args.tp_share.split(",") if v]:
        if K % (64 * P) != 0 or T % P != 0:
            log(f"P={P}: K/P or T/P is not a whole number of 64-column groups / rows; skipped")
            continue
        kp = K // P
        for mc in (T, 512):
            n_chunks = T // mc
            # projection share: one chunk of mc tokens over K/P columns into one fp32 partial
            # (K split 1), and as the library would run it (its own tile and K split; the
            # split partials would be summed before the exchange)
            d, x, Wp, r, w, out = device_inputs(mc, kp)
            call = lambda: pr.proj_add_rmsnorm(x, Wp, r, w, d["eps"], mc, kp, H, mc, wl.norm_kind,
                                               out)
            auto_split = pr.pr_select(mc, kp, H, mc)["split_k"]
            t_auto = per_launch(call, "gemm")
            y_part = torch.empty((P, mc, H), dtype=torch.float32, device=dev)
            t_proj = per_launch(lambda: pr.pr_project_partial(x, Wp, y_part[0], mc, kp, H),
                                "gemm")
            # add/norm share: the owner's mc/P rows summing the P fp32 partials in rank order
            rows = mc // P
            t_an = per_launch(lambda: pr.pr_add_rmsnorm_partials(y_part, P, mc * H, r, w,
                                                                 d["eps"], rows, H, wl.norm_kind,
                                                                 out), "addnorm")
            del y_part
            rs_fp32 = (P - 1) and rows * H * 4 / (XGMI_LINK_GBS * 1e3)  # us per link
            rs_bf16 = (P - 1) and rows * H * 2 / (XGMI_LINK_GBS * 1e3)
            ag_bf16 = (P - 1) and rows * H * 2 / (XGMI_LINK_GBS * 1e3)
            serial = t_proj + rs_fp32 + t_an + ag_bf16
            overlapped = max(t_proj, rs_fp32, t_an, ag_bf16)
            row = {"P": P, "mc": mc, "chunks": n_chunks, "K_share": kp, "rows_share": rows,
                   "proj_share_us": t_proj, "addnorm_share_us": t_an,
                   "proj_share_tflops": 2.0 * mc * kp * H / t_proj / 1e6,
                   "proj_share_auto_us": t_auto, "proj_share_auto_split": auto_split,
                   "addnorm_share_gbs": rows * H * (4 * P + 10) / t_an / 1e3,
                   "rs_fp32_model_us": rs_fp32, "rs_bf16_model_us": rs_bf16,
                   "ag_bf16_model_us": ag_bf16,
                   "per_chunk_serial_us": serial, "per_chunk_overlapped_bound_us": overlapped,
                   "call_serial_us": serial * n_chunks,
                   "call_pipelined_bound_us": (overlapped * n_chunks + serial - overlapped
                                               if n_chunks > 1 else serial)}
            rows_out.append(row)
            log(f"P={P} mc={mc}: proj share {t_proj:.1f} us (library's choice, split "
                f"{auto_split}: {t_auto:.1f} us), add/norm share {t_an:.1f} us, "
                f"RS fp32 {rs_fp32:.1f} / AG bf16 {ag_bf16:.1f} us (model)")
    print(json.dumps({"tp_share": {"workload": wl.name, "T": T, "K": K, "H": H,
                                   "xgmi_link_GBs": XGMI_LINK_GBS, "rows": rows_out}}),
          flush=True)
    return 0


def phases(pr, torch, args) -> int:
    """In-kernel phase and clock stamps of the single launch on each workload (the diagnostic
    library, selected by PR_PHASE_STAMPS=1 before the first library call).  A workload named
    W:fp8 runs the FP8 single launch (activations quantised once, 256-token scale groups)."""
    import synth
    from projection_residual_rmsnorm_amd import profiling
    results = {}
    dev = "cuda:0"
    for spec in args.phases.split(","):
        name, _, form = spec.partition(":")
        fp8 = form == "fp8"
        wl = synth.WORKLOADS[name]
        T, K, H = wl.T, wl.K, wl.H
        d = synth.make_inputs(wl, seed=0)
        x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
        W_src = torch.from_numpy(d["W"].view(np.int16)).to(dev)
        r = torch.from_numpy(d["residual"]).to(dev)
        w = torch.from_numpy(d["norm_w"]).to(dev)
        out = torch.empty((T, H), dtype=torch.int16, device=dev)
        stream = torch.cuda.Stream()
        if fp8:
            scale_rows = 256
            wq = torch.empty((H, K), dtype=torch.uint8, device=dev)
            sw = torch.empty(1, dtype=torch.float32, device=dev)
            pr.pr_quantize_fp8(W_src, wq, sw, H, K, H, stream)
            Wp = torch.empty(K * H, dtype=torch.uint8, device=dev)
            pr.pr_prepare_weight_fp8(wq, pr.PR_WEIGHT_OUT_IN, Wp, K, H, stream)
            xq = torch.empty((T, K), dtype=torch.uint8, device=dev)
            sx = torch.empty(((T - 1) // scale_rows + 1,), dtype=torch.float32, device=dev)
            pr.pr_quantize_fp8(x, xq, sx, T, K, scale_rows, stream)
            call = lambda: pr.proj_add_rmsnorm_fp8(xq, sx, scale_rows, Wp, sw, r, w, d["eps"], T,
                                                   K, H, wl.norm_kind, out, stream)
        else:
            Wp = torch.empty(K * H, dtype=torch.int16, device=dev)
            pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
            call = lambda: pr.proj_add_rmsnorm_single_launch(x, Wp, r, w, d["eps"], T, K, H,
                                                             wl.norm_kind, out, stream=stream)
        torch.cuda.synchronize()
        assert pr.loaded_library_path() == pr.STAMPS_LIB_PATH, pr.loaded_library_path()
        # The FP8 launch takes the bf16 single launch's tile, with 8 waves, in two K groups
        # where the bf16 launch uses them and K holds whole 128-deep stages; for the bf16-only
        # 192 x 192 tile it takes the one of the other tiles whose one-round grid has as many
        # workgroups as the launch stamps.
        c = pr.pr_select(T, K, H, pr.PR_SINGLE_LAUNCH)
        bm, bn = c["gemm_bm"], c["gemm_bn"]
        waves = 8 if fp8 else c["gemm_waves"]
        kgroups = c["gemm_kgroups"] if not fp8 or K % 128 == 0 else 1
        for _ in range(max(args.warmup, 1)):
            call()
        if fp8 and (bm, bn) == (192, 192):
            pr.pr_phase_stamps(clear=True)
            call()
            n_wg = int(np.count_nonzero(pr.pr_phase_stamps()[:, 1]))
            bm, bn = next(((m, n) for m, n in ((256, 256), (256, 128), (128, 128))
                           if H % n == 0 and -(-T // m) * (H // n) == n_wg), (bm, bn))
            kgroups = 2 if (bm, bn) == (256, 128) and K % 128 == 0 else 1
        cfg = (f"{bm}x{bn} tiles, {waves} waves"
               + (f" in {kgroups} K groups" if kgroups > 1 else ""))
        tiles = -(-T // bm) * (H // bn)
        trials = []
        for _ in range(5):
            pr.pr_phase_stamps(clear=True)
            for _ in range(3):
                call()
            a = pr.pr_phase_stamps()  # synchronises the device
            a = a[a[:, 1] != 0]
            # the matrix cores' share is derived only for one-round grids (every workgroup one
            # whole tile)
            fpg = 2.0 * bm * bn * K if a.shape[0] == tiles else 0.0
            trials.append(profiling.phase_stats(a, fpg, 8192.0 if fp8 else 4096.0))
        assert pr.pr_device_status(stream) == 0
        results[spec] = {"shape": f"T={T}, K={K}, H={H}" + (", FP8 E4M3" if fp8 else ""),
                         "config": cfg, "trials": trials,
                         "rounds": -(-tiles // trials[0]["workgroups"])}
        ph = trials[-1]["phases_us"]
        log(f"{spec}: main loop {ph[0]:.1f} us at {trials[-1]['clock_mhz']:.0f} MHz, "
            f"span {trials[-1]['span_us']:.1f} us")
    # The command as run from the repository root (the output path made relative to it).
    argv = [os.path.relpath(a, ROOT) if os.path.isabs(a) and a.startswith(ROOT) else a
            for a in sys.argv[1:]]
    text = profiling.phases_summary(results, "python bench.py " + " ".join(argv))
    if args.phases_out:
        with open(args.phases_out, "w") as f:
            f.write(text)
    else:
        print(text)
    return 0


def main() -> int:
    args = parse()
    if args.phases:
        # the diagnostic library with in-kernel stamps (selected before any library call)
        os.environ["PR_PHASE_STAMPS"] = "1"
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              "inter-GPU step", file=sys.stderr)
        return 2
    clocks = clock_settings()  # before this process touches the GPU
    import torch
    import projection_residual_rmsnorm_amd as pr
    import synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.phases:
        return phases(pr, torch, args)
    if args.tune_sweep:
        return tune_sweep(pr, torch, args)
    if args.tp_share:
        return tp_share(pr, torch, args)
    if args.cu_split:
        return cu_split_table(pr, torch, args)
    if args.addnorm_roofline:
        return addnorm_roofline(pr, torch, args)
    if args.silu_mul:
        return silu_mul_roofline(pr, torch, args)
    wl = synth.WORKLOADS[args.workload]
    T, K, H = wl.T, wl.K, wl.H
    log(f"workload {wl.name}: T={T} K={K} H={H} chunk sizes {wl.microchunks}")
    d = synth.make_inputs(wl, seed=0)
    dev = "cuda:0"
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    W_src = torch.from_numpy(d["W"].view(np.int16)).to(dev)
    Wp = torch.empty(K * H, dtype=torch.int16, device=dev)
    pr.pr_prepare_weight(W_src, pr.PR_WEIGHT_OUT_IN, Wp, K, H)
    r = torch.from_numpy(d["residual"]).to(dev)
    w = torch.from_numpy(d["norm_w"]).to(dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    # All timed work runs on one dedicated stream (the legacy null stream adds host-side
    # synchronisation to every event record on it).
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    flops = 2.0 * T * K * H

    def fused(mc):
        if mc == "single":
            return lambda: pr.proj_add_rmsnorm_single_launch(x, Wp, r, w, d["eps"], T, K, H,
                                                             wl.norm_kind, out)
        return lambda: pr.proj_add_rmsnorm(x, Wp, r, w, d["eps"], T, K, H, mc, wl.norm_kind, out)

    def conventional():
        pr.proj_add_rmsnorm_unfused(x, Wp, r, w, d["eps"], T, K, H, wl.norm_kind, out)

    mcs = [args.microchunk] if args.microchunk else list(wl.microchunks)
    # The library's load-time tuning for this shape group (untimed): it picks the projection
    # configuration of each chunk size (checked against the conventional path) and a token
    # threshold for auto mode.  Explicit-chunk calls below use the tuned configurations.
    chunk_cfgs = {}
    if not args.no_tune:
        t_tune = time.perf_counter()
        rep = pr.pr_tune([K], [H], wl.norm_kind, [T], mcs, reps=5, stream=stream)
        log(f"tuned in {time.perf_counter() - t_tune:.1f} s (checked {rep['n_checked']}, "
            f"rejected {rep['n_rejected']})")
    # The configuration each fused form runs with (tuned, or the time model's without tuning;
    # the single launch's does not depend on tuning).
    for m in mcs + [pr.PR_SINGLE_LAUNCH]:
        c = pr.pr_select(T, K, H, m)
        chunk_cfgs["single" if m == pr.PR_SINGLE_LAUNCH else str(m)] = (
            f"{c['gemm_bm']}x{c['gemm_bn']} split {c['split_k']} {c['gemm_waves']} waves"
            + (f" {c['gemm_kgroups']} K groups" if c["gemm_kgroups"] > 1 else "")
            + (f" CU split {c['addnorm_cus']}" if c["addnorm_cus"] > 0 else ""))
    log(f"configurations: {chunk_cfgs}")
    per_mc = {}
    if args.only_single:
        forms = ["single"]
    else:
        forms = mcs + (["single"] if not args.microchunk else [])
    for mc in forms:
        el = time_steps(fused(mc), args.steps, args.warmup, torch)
        per_mc[mc] = {"tokens_per_s": T * args.steps / el, "ms_per_step": el * 1e3 / args.steps,
                      "tflops": flops * args.steps / el / 1e12}
        log(f"fused {'single launch' if mc == 'single' else f'mc={mc}'}: "
            f"{per_mc[mc]['ms_per_step']:.4f} ms/step {per_mc[mc]['tflops']:.1f} TFLOP/s")
    if "single" in per_mc and pr.pr_device_status(stream) != 0:
        raise SystemExit("single-launch status bits set: a row wait gave up")
    best = min(per_mc, key=lambda m: per_mc[m]["ms_per_step"])
    el_c = time_steps(conventional, args.steps, args.warmup, torch)
    conv = {"tokens_per_s": T * args.steps / el_c, "ms_per_step": el_c * 1e3 / args.steps,
            "tflops": flops * args.steps / el_c / 1e12}
    log(f"conventional: {conv['ms_per_step']:.4f} ms/step {conv['tflops']:.1f} TFLOP/s")

    # Headline: the fastest fused form, timed as its own region (barrier-free single process:
    # synchronize on both sides).
    mc = best
    el = time_steps(fused(mc), args.steps, args.warmup, torch)
    value = T * args.steps / el
    ms_step = el * 1e3 / args.steps
    tflops = flops * args.steps / el / 1e12

    # Kernel durations: the same steps again with the library's timing events bracketing every
    # projection and add/norm launch on the stream it runs on.
    pr.pr_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fused(mc)()
    torch.cuda.synchronize()
    el_prof = time.perf_counter() - t0
    prof = pr.pr_profile_read()
    pr.pr_profile_enable(False)

    single = mc == "single"
    if single and pr.pr_device_status(stream) != 0:
        raise SystemExit("single-launch status bits set: a row wait gave up")
    g_launch_s = prof["gemm_ms"] / max(prof["gemm_launches"], 1) / 1e3
    gemm_flops_per_launch = flops * args.steps / max(prof["gemm_launches"], 1)
    gemm_tflops = gemm_flops_per_launch / g_launch_s / 1e12
    split = pr.pr_select(T, K, H, pr.PR_SINGLE_LAUNCH if single else mc)["split_k"]
    if single:
        # One kernel per call: its HBM bytes beyond the projection are the residual read and
        # write and the output write (10 B per element).
        a_launch_s, addnorm_bytes_per_elem, addnorm_gbs = None, 10, None
    else:
        a_launch_s = prof["addnorm_ms"] / max(prof["addnorm_launches"], 1) / 1e3
        addnorm_elems_per_launch = T * H * args.steps / max(prof["addnorm_launches"], 1)
        addnorm_bytes_per_elem = 4 * split + 4 + 4 + 2   # slot planes + r read + r write + out
        addnorm_gbs = addnorm_elems_per_launch * addnorm_bytes_per_elem / a_launch_s / 1e9
    # Measured HBM bytes per projection launch, from the committed counter runs; null unless
    # they were taken on this exact kernel source and this workload / chunk size.
    traffic = None
    if args.traffic_dir and os.path.isdir(args.traffic_dir):
        import glob
        from projection_residual_rmsnorm_amd.profiling import source_digest
        src = os.path.join(ROOT, "projection_residual_rmsnorm_amd", "csrc", "pr_kernels.hip")
        digest, label = source_digest(src), traffic_label(wl.name, mc, chunk_cfgs)
        for path in sorted(glob.glob(os.path.join(args.traffic_dir, "traffic_*.json"))):
            with open(path) as f:
                tr = json.load(f)
            if tr.get("kernel_source_sha256") == digest and tr.get("config") == label:
                traffic = tr.get("gemm_bytes_per_launch")
    roof = {"kernel": "gemm_add_rmsnorm_kernel" if single else "gemm_bf16_kernel",
            "bound": "mfma", "achieved": gemm_tflops,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": gemm_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic, "avg_launch_us": g_launch_s * 1e6,
            "launches": prof["gemm_launches"], "flops_per_launch": gemm_flops_per_launch,
            "timed_pass_ms_per_step": el_prof * 1e3 / args.steps}
    kernels = {"gemm_avg_us": g_launch_s * 1e6, "gemm_tflops": gemm_tflops,
               "addnorm_avg_us": None if a_launch_s is None else a_launch_s * 1e6,
               "addnorm_gbs": addnorm_gbs,
               "addnorm_bytes_per_elem": addnorm_bytes_per_elem, "split_k": split}
    result = {
        "metric": "fused proj+add+RMSNorm tokens/s; TFLOP/s as % bf16 MFMA peak (1 GPU)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name} prefill", "T": T, "K": K, "H": H,
                   "microchunk": None if single else mc,
                   "norm": "gemma" if wl.norm_kind else "standard",
                   "path": "fused single launch" if single else "fused microchunk pipeline",
                   "parallelism": "none (1 GPU)"},
        "tflops": tflops, "frac_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "roofline": roof, "kernels": kernels,
        "per_microchunk": {str(k): v for k, v in per_mc.items()},
        "chunk_configs": chunk_cfgs,
        "conventional": conv,
        "clocks": clocks,
    }
    # Per-call statistics of the headline form and the conventional path: residual restored
    # before every call; warm (operands may sit in the Infinity Cache) and flushed.  Not in
    # profiler runs (--only-single), whose kernel averages must match the timed region.
    if args.only_single:
        result["per_call"] = None
    else:
        add_per_call_stats(result, fused(mc), conventional, r, args.steps, torch, stream, dev,
                           "single launch" if single else f"mc={mc}")
    # The conventional add/norm with cold caches (the HBM-bound stage) and the second
    # 4096-class shape; not in profiler runs (--only-single).
    if not args.only_single:
        result["addnorm_conventional"] = conventional_addnorm_flushed(
            pr, torch, x, Wp, r, w, out, d, wl, args.steps, stream)
        result["fp8"] = fp8_entry(pr, torch, x, W_src, r, w, out, d, wl.norm_kind,
                                  min(wl.microchunks), args, stream)
        if wl.name == "o_proj":
            result["down_proj"] = down_proj_entry(pr, torch, args, stream)
            # the fused-or-conventional crossover of the long-prefill sweep (a few seconds; it
            # tunes, so not with --no-tune, which the profiled runs pass: the tuner's CU-masked
            # streams make rocprofv3 crash in its exit handler before it writes its files)
            if not args.no_tune:
                result["threshold_sweep"] = threshold_sweep(pr, args)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    del W_src
    if not args.no_cpu_baseline:
        log(f"timing the oracle on the host for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
