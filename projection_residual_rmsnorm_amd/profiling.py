"""Summaries of rocprofv3 CSV output for the kernels of this library.

    python -m projection_residual_rmsnorm_amd.profiling stats <kernel_stats.csv> <out.md> \
        --command "<the rocprofv3 command that produced it>" \
        [--trace <kernel_trace.csv> --kernel "<kernel name prefix>" --last N]
        [--bench-log <stdout of the profiled bench.py>]
    python -m projection_residual_rmsnorm_amd.profiling traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> --kernel "<kernel name prefix>" --out <traffic.json> \
        --command "<commands>"

    python -m projection_residual_rmsnorm_amd.profiling counters <counter_collection.csv> <out.md> \
        --kernel "<kernel name prefix>" [--kernel ...] [--grid N] --command "<command>"

    python -m projection_residual_rmsnorm_amd.profiling runs <kernel_trace.csv> <out.md> \
        --kernel "<kernel name prefix>" --per-run N --labels "a,b,..." --command "<command>"

`phases_summary` turns the in-kernel phase stamps of the diagnostic library (read by
`bench.py --phases`) into a markdown table.

`traffic` calibrates FETCH_SIZE and WRITE_SIZE (KiB per dispatch) against the plain 1 GiB
device copies that `bench.py --copy-calibration` runs in the same process: the factor that
turns each counter into bytes is (1 GiB) / (the counter's reading for one such copy).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import re
import statistics
from typing import Dict, List

COPY_BYTES = 1 << 30


def short_name(name: str) -> str:
    m = re.search(r"(gemm_add_rmsnorm_kernel<[^>]*>|gemm_bf16_kernel<[^>]*>|"
                  r"(?<!gemm_)add_rmsnorm\w*<[^>]*>|add_rmsnorm_generic_kernel|"
                  r"prepare_weight\w*|silu_mul_kernel<[^>]*>|__amd_rocclr_\w+|fill_\w+|"
                  r"delay_kernel)", name)
    return m.group(1) if m else name[:60]


def stats_summary(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | average us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(lines) + "\n"


def last_dispatches(trace_csv: str, kernel: str, n: int) -> dict:
    """Durations of the last n dispatches of a kernel (name prefix) in a kernel-trace CSV, in
    dispatch order: the pass a bench run times with events when that pass ends the program."""
    durs = []
    for r in csv.DictReader(open(trace_csv)):
        if short_name(r["Kernel_Name"]).startswith(kernel):
            durs.append((int(r["Dispatch_Id"]),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    if len(durs) < n:
        raise SystemExit(f"kernel {kernel!r}: {len(durs)} dispatches in the trace, asked for {n}")
    last = [d for _, d in sorted(durs)[-n:]]
    return {"kernel": kernel, "n": n, "mean_us": statistics.mean(last),
            "median_us": statistics.median(last), "min_us": min(last), "max_us": max(last)}


def last_pass_lines(res: dict) -> List[str]:
    return ["", f"Last {res['n']} dispatches of `{res['kernel']}` (the bench's event-timed pass): "
                f"mean {res['mean_us']:.2f} us, median {res['median_us']:.2f}, "
                f"min {res['min_us']:.2f}, max {res['max_us']:.2f}."]


def bench_line_lines(log_path: str) -> List[str]:
    """The roofline figures of the bench line printed by the profiled program itself."""
    line = [l for l in open(log_path) if l.startswith("{")][-1]
    roof = json.loads(line)["roofline"]
    return ["", f"The bench line of the same run: `{roof['kernel']}` averaged "
                f"{roof['avg_launch_us']:.2f} us over {roof['launches']} event-timed launches "
                f"({roof['achieved']:.1f} {roof['unit']})."]


def dispatch_runs(trace_csv: str, kernel: str, n, labels: List[str]) -> List[dict]:
    """Consecutive runs of dispatches of a kernel (name prefix) in dispatch order, one per
    label, with their median, min and max durations in us; n is the dispatch count of every
    run, or a list with one count per run."""
    counts = list(n) if isinstance(n, (list, tuple)) else [n] * len(labels)
    if len(counts) != len(labels):
        raise SystemExit(f"{len(counts)} run lengths for {len(labels)} labels")
    durs = []
    for r in csv.DictReader(open(trace_csv)):
        if short_name(r["Kernel_Name"]).startswith(kernel):
            durs.append((int(r["Dispatch_Id"]),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    durs = [d for _, d in sorted(durs)]
    if len(durs) != sum(counts):
        raise SystemExit(f"kernel {kernel!r}: {len(durs)} dispatches, expected {sum(counts)}")
    out, at = [], 0
    for label, c in zip(labels, counts):
        run = durs[at:at + c]
        at += c
        out.append({"label": label, "n": c, "median_us": statistics.median(run),
                    "min_us": min(run), "max_us": max(run)})
    return out


def runs_summary(trace_csv: str, kernel: str, n, labels: List[str], command: str) -> str:
    lines = ["# rocprofv3 kernel trace: runs of dispatches", "", "Command:", "", "```", command,
             "```", "", f"Kernel `{kernel}`, consecutive runs of dispatches in dispatch order.",
             "",
             "| run | dispatches | median us | min us | max us |", "|---|---|---|---|---|"]
    for r in dispatch_runs(trace_csv, kernel, n, labels):
        lines.append(f"| {r['label']} | {r['n']} | {r['median_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} |")
    return "\n".join(lines) + "\n"


def _counter(path: str, counter: str, grid: int = 0) -> Dict[str, List[float]]:
    """Counter values per kernel; with grid > 0, only dispatches of that grid size (threads) for
    kernels other than the calibration copies (one kernel can serve several launch shapes)."""
    out: Dict[str, List[float]] = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = short_name(r["Kernel_Name"])
        if grid and not name.startswith("__amd_rocclr") and int(r["Grid_Size"]) != grid:
            continue
        out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_csv: str, write_csv: str, kernel: str, grid: int = 0) -> dict:
    fetch = _counter(fetch_csv, "FETCH_SIZE", grid)
    write = _counter(write_csv, "WRITE_SIZE", grid)
    big = lambda vals: [v for v in vals if v * 1024 > COPY_BYTES / 4]
    copy_f = big(fetch.get("__amd_rocclr_copyBuffer", []))
    copy_w = big(write.get("__amd_rocclr_copyBuffer", []))
    if not copy_f or not copy_w:
        raise SystemExit("no 1 GiB copy dispatches found (run bench.py with --copy-calibration)")
    f_factor = COPY_BYTES / (statistics.median(copy_f) * 1024)
    w_factor = COPY_BYTES / (statistics.median(copy_w) * 1024)
    kf = [v for k, vals in fetch.items() if k.startswith(kernel) for v in vals]
    kw = [v for k, vals in write.items() if k.startswith(kernel) for v in vals]
    if not kf or not kw:
        raise SystemExit(f"kernel {kernel!r} not found in the counter files")
    fetched = statistics.mean(kf) * 1024 * f_factor
    written = statistics.mean(kw) * 1024 * w_factor
    return {"kernel": kernel, "grid_size": grid, "dispatches": len(kf),
            "fetch_size_kib_mean": statistics.mean(kf), "write_size_kib_mean": statistics.mean(kw),
            "copy_fetch_size_kib": statistics.median(copy_f),
            "copy_write_size_kib": statistics.median(copy_w),
            "fetch_factor": f_factor, "write_factor": w_factor,
            "fetched_bytes_per_launch": fetched, "written_bytes_per_launch": written,
            "gemm_bytes_per_launch": fetched + written}


CU_COUNT = 256
SIMDS_PER_CU = 4
MOP_FLOPS = 512  # SQ_INSTS_VALU_MFMA_MOPS_*: one count per 512 floating-point operations


def counter_table(path: str, kernels: List[str], grid: int = 0) -> Dict[str, dict]:
    """Per kernel (name prefix), the mean of every collected counter over its dispatches, and
    the dispatch duration when the file has timestamps (a run with --kernel-trace)."""
    per: Dict[str, Dict[int, dict]] = {}
    for r in csv.DictReader(open(path)):
        name = short_name(r["Kernel_Name"])
        k = next((k for k in kernels if name.startswith(k)), None)
        if k is None or (grid and int(r["Grid_Size"]) != grid):
            continue
        d = per.setdefault(k, {}).setdefault(int(r["Dispatch_Id"]), {"name": name})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            d["duration_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for k, disp in per.items():
        names = sorted({c for d in disp.values() for c in d if c != "name"})
        out[k] = {"kernel": sorted({d["name"] for d in disp.values()}),
                  "dispatches": len(disp),
                  "mean": {c: statistics.mean(d[c] for d in disp.values() if c in d)
                           for c in names}}
    return out


NAMEPLATE_GHZ = 2.4
XCDS = 8
SHADER_ENGINES = 32  # 4 per XCD


def derived(mean: Dict[str, float]) -> Dict[str, float]:
    """Ratios the counters support.

    SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs; one 32x32x16 bf16 MFMA keeps a SIMD
    busy 32 cycles, so for a bf16 kernel the sum is the instruction count x 32, i.e. flops /
    1024: it restates the flop count and is not reported as a separate utilisation.
    GRBM_GUI_ACTIVE spans the counter window, which is longer than the dispatch (several times
    longer for a kernel of a few microseconds), so it gives no clock and is not used.
      shader_clock_GHz_busy: SQ_BUSY_CYCLES (shader-clock cycles with waves present, summed
        over the 32 shader engines) / (32 x duration).  An engine without waves for part of
        the dispatch (the last workgroups' tail) lowers it, so it is a lower bound of the clock;
      shader_clock_GHz_cycles: SQ_CYCLES / (32 x duration), over the counter window, which is
        longer than the dispatch: an upper bound;
      mfma_util_at_busy_clock: MFMA busy cycles / (SIMDs x duration x the lower-bound clock),
        so an upper bound of the matrix cores' busy fraction at the clock the kernel ran at;
      lds_bank_conflict_frac: conflict cycles / LDS-active cycles;
      l1_l2_read_MB_at_64B: L1 -> L2 read requests x 64 bytes;
      l1_l2_read_latency_cycles: summed request latency / requests;
      l1_pending_stall_cycles_per_cu: cycles an L1 waited on data pending from L2, per CU."""
    out = {}
    simds = CU_COUNT * SIMDS_PER_CU
    busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES")
    dur = mean.get("duration_ns")
    if dur:
        out["duration_us"] = dur / 1e3
    if mean.get("SQ_BUSY_CYCLES") and dur:
        clk = mean["SQ_BUSY_CYCLES"] / SHADER_ENGINES / dur
        out["shader_clock_GHz_busy"] = clk
        if busy is not None:
            out["mfma_util_at_busy_clock"] = busy / (simds * dur * clk)
    if mean.get("SQ_CYCLES") and dur:
        out["shader_clock_GHz_cycles"] = mean["SQ_CYCLES"] / SHADER_ENGINES / dur
    req = mean.get("TCP_TCC_READ_REQ_sum")
    if req:
        out["l1_l2_read_MB_at_64B"] = req * 64 / 1e6
        if "TCP_TCC_READ_REQ_LATENCY_sum" in mean:
            out["l1_l2_read_latency_cycles"] = mean["TCP_TCC_READ_REQ_LATENCY_sum"] / req
    if "TCP_PENDING_STALL_CYCLES_sum" in mean:
        out["l1_pending_stall_cycles_per_cu"] = mean["TCP_PENDING_STALL_CYCLES_sum"] / CU_COUNT
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean:
        out["mfma_bf16_flops"] = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * MOP_FLOPS
        if dur:
            out["mfma_bf16_TFLOPs"] = out["mfma_bf16_flops"] / dur / 1e3
    if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_LDS_IDX_ACTIVE"):
        out["lds_bank_conflict_frac"] = mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_LDS_IDX_ACTIVE"]
    return out


def counters_summary(path: str, kernels: List[str], grid: int, command: str) -> str:
    tab = counter_table(path, kernels, grid)
    lines = ["# rocprofv3 counters per dispatch", "", "Command:", "", "```", command, "```", ""]
    for k in kernels:
        if k not in tab:
            lines += [f"`{k}`: no dispatches in the file", ""]
            continue
        t = tab[k]
        lines += [f"## `{', '.join(t['kernel'])}` ({t['dispatches']} dispatches)", "",
                  "| counter | mean per dispatch |", "|---|---|"]
        lines += [f"| {c} | {v:.6g} |" for c, v in t["mean"].items()]
        dv = derived(t["mean"])
        if dv:
            lines += ["", "| derived | value |", "|---|---|"]
            lines += [f"| {c} | {v:.4g} |" for c, v in dv.items()]
        lines.append("")
    return "\n".join(lines)


def _code_only(text: str) -> str:
    """The source without comments, whitespace runs collapsed (string and character literals
    are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


PHASES = ["main loop", "K groups' hand-over", "staging: r + y and row sums", "publish",
          "row wait", "slot reads", "residual and output stores acknowledged"]


def phase_stats(trial, flops_per_group: float = 0.0, flops_per_clock: float = 4096.0) -> dict:
    """One launch's stamps (rows: workgroups of round 0; words as pr_phase_stamps documents)
    reduced to medians over workgroups.  Times in µs from the 100 MHz constant clock; the main
    loop's shader clock in MHz; with flops_per_group, the matrix cores' busy fraction of the
    main loop at that clock (flops_per_clock dense flops per CU and clock: 4096 for bf16, 8192
    for fp8)."""
    import numpy as np
    a = np.asarray(trial, dtype=np.uint64)
    rt = a[:, 1:9].astype(np.int64)
    t = (rt - rt[:, 0].min()) / 100.0
    dur = np.diff(t, axis=1)
    clock = (a[:, 11].astype(np.int64) - a[:, 10].astype(np.int64)) / dur[:, 0]
    res = {
        "workgroups": int(a.shape[0]),
        "phases_us": [float(np.median(dur[:, p])) for p in range(dur.shape[1])],
        "clock_mhz": float(np.median(clock)),
        "clock_mhz_p10_p90": [float(np.percentile(clock, 10)), float(np.percentile(clock, 90))],
        "span_us": float(t[:, 7].max()),
        "main_loop_end_spread_us": float(t[:, 1].max() - t[:, 1].min()),
        "after_last_main_loop_us": float(t[:, 7].max() - t[:, 1].max()),
        "xcd": {},
    }
    if flops_per_group:
        busy = flops_per_group / (flops_per_clock * clock * 1e6 * dur[:, 0] * 1e-6)
        res["mfma_busy_main_loop"] = float(np.median(busy))
        res["flops_per_clock"] = flops_per_clock
    xcc = a[:, 0].astype(int)
    for x in sorted(set(xcc.tolist())):
        m = xcc == x
        res["xcd"][x] = {"main_loop_us": float(np.median(dur[m, 0])),
                         "clock_mhz": float(np.median(clock[m])),
                         "main_loop_end_us": [float(t[m, 1].min()), float(t[m, 1].max())]}
    return res


def phases_summary(results: Dict[str, dict], command: str) -> str:
    """results: workload -> {"shape": str, "config": str, "rounds": int (tile rounds of the
    launch; only the first is stamped), "trials": [phase_stats(...), ...]}."""
    import numpy as np
    lines = ["# Single launch: in-kernel phase and clock stamps", "",
             f"Command: `{command}`", "",
             "Thread 0 of every workgroup stamps the constant 100 MHz clock at each phase "
             "boundary of the single launch, and the shader clock around the main loop "
             "(`libprojaddnorm_stamps.so`, the default sources compiled with "
             "`PR_PHASE_STAMPS`). Each trial is the last of three back-to-back calls. Per "
             "phase: the median over the launch's workgroups, as the median over trials [min–max "
             "over trials], µs.", ""]
    for name, r in results.items():
        tr = r["trials"]
        lines += [f"## {name}: {r['shape']}, {r['config']}", "",
                  "| phase | µs |", "|---|---|"]
        for p, ph in enumerate(PHASES):
            v = [x["phases_us"][p] for x in tr]
            lines.append(f"| {ph} | {np.median(v):.1f} [{min(v):.1f}–{max(v):.1f}] |")

        def agg(key, fmt=".1f"):
            v = [x[key] for x in tr]
            return f"{np.median(v):{fmt}} [{min(v):{fmt}}–{max(v):{fmt}}]"
        rounds = r.get("rounds", 1)
        span = ("launch span" if rounds == 1 else
                f"span of the first of {rounds} rounds (only it is stamped)")
        lines += ["", f"- workgroups stamped per launch: {tr[0]['workgroups']}",
                  f"- {span}, first start to last stores acknowledged: {agg('span_us')} µs",
                  f"- spread of main-loop end times over workgroups: "
                  f"{agg('main_loop_end_spread_us')} µs",
                  f"- last stores acknowledged after the slowest main loop: "
                  f"{agg('after_last_main_loop_us')} µs",
                  f"- shader clock during the main loop: {agg('clock_mhz')} MHz (median over "
                  f"workgroups; p10–p90 of the last trial "
                  f"{tr[-1]['clock_mhz_p10_p90'][0]:.0f}–{tr[-1]['clock_mhz_p10_p90'][1]:.0f})"]
        if "mfma_busy_main_loop" in tr[0]:
            lines.append(f"- matrix cores busy during the main loop, at that clock: "
                         f"{agg('mfma_busy_main_loop', '.2f')} (fraction; "
                         f"flops per workgroup ÷ ({tr[0]['flops_per_clock']:.0f} × clock × "
                         "main-loop time))")
        lines += ["", "Per XCD, last trial:", "",
                  "| XCC | main loop µs | clock MHz | main loops end at µs |", "|---|---|---|---|"]
        for x, v in tr[-1]["xcd"].items():
            lines.append(f"| {x} | {v['main_loop_us']:.1f} | {v['clock_mhz']:.0f} | "
                         f"{v['main_loop_end_us'][0]:.1f}–{v['main_loop_end_us'][1]:.1f} |")
        lines.append("")
    return "\n".join(lines)


def _without_stamps(text: str) -> str:
    """The source without its diagnostic phase stamps: every #ifdef PR_PHASE_STAMPS block
    (both branches: the stamp code, and the no-op PR_PHASE macro of the default build) and the
    PR_PHASE(n) statements removed.  The default library's code is what remains."""
    out, depth = [], 0  # depth > 0: inside a PR_PHASE_STAMPS block (counting nested #ifs)
    for line in text.splitlines():
        d = line.strip()
        if depth:
            if d.startswith("#if"):
                depth += 1
            elif d.startswith("#endif"):
                depth -= 1
            continue
        if d == "#ifdef PR_PHASE_STAMPS":
            depth = 1
            continue
        out.append(line)
    return re.sub(r"\bPR_PHASE\(\d+\);", "", "\n".join(out))


def source_digest(path: str) -> str:
    """sha256 of a kernel source file's code as the default library compiles it (comments,
    whitespace and the diagnostic phase stamps do not count): counter readings are void once
    the kernels' code changes."""
    return hashlib.sha256(_code_only(_without_stamps(open(path).read())).encode()).hexdigest()


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--trace", help="kernel_trace.csv of the same run")
    s.add_argument("--kernel", help="kernel name prefix for the last-pass figure")
    s.add_argument("--last", type=int, default=0, help="dispatches in the last timed pass")
    s.add_argument("--bench-log", help="stdout of the profiled bench.py (its JSON line)")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--kernel", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--config", required=True, help="workload label, e.g. o_proj:mc=512")
    t.add_argument("--source", required=True, help="kernel source the counters were taken on")
    t.add_argument("--grid", type=int, default=0,
                   help="only dispatches of this grid size (threads), e.g. one chunk's launch")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--grid", type=int, default=0)
    c.add_argument("--command", required=True)
    u = sub.add_parser("runs")
    u.add_argument("trace")
    u.add_argument("out")
    u.add_argument("--kernel", required=True)
    u.add_argument("--per-run", required=True,
                   help="dispatches per run: one count, or one per label (comma-separated)")
    u.add_argument("--labels", required=True, help="comma-separated, one per run")
    u.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "runs":
        with open(a.out, "w") as f:
            counts = [int(c) for c in a.per_run.split(",")]
            f.write(runs_summary(a.trace, a.kernel, counts if len(counts) > 1 else counts[0],
                                 a.labels.split(","), a.command))
    elif a.cmd == "counters":
        with open(a.out, "w") as f:
            f.write(counters_summary(a.csv, a.kernel, a.grid, a.command))
    elif a.cmd == "stats":
        with open(a.out, "w") as f:
            f.write(stats_summary(a.csv, a.command))
            if a.trace and a.kernel and a.last:
                f.write("\n".join(last_pass_lines(last_dispatches(a.trace, a.kernel, a.last)))
                        + "\n")
            if a.bench_log:
                f.write("\n".join(bench_line_lines(a.bench_log)) + "\n")
    else:
        res = traffic(a.fetch_csv, a.write_csv, a.kernel, a.grid)
        res["commands"] = a.command
        res["config"] = a.config
        res["kernel_source_sha256"] = source_digest(a.source)
        with open(a.out, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main()
