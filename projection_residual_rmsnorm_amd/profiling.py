"""Summaries of rocprofv3 CSV output for the kernels of this library.

    python -m projection_residual_rmsnorm_amd.profiling stats <kernel_stats.csv> <out.md> \
        --command "<the rocprofv3 command that produced it>"
    python -m projection_residual_rmsnorm_amd.profiling traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> --kernel "<kernel name prefix>" --out <traffic.json> \
        --command "<commands>"

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
                  r"prepare_weight\w*|__amd_rocclr_\w+|fill_\w+|delay_kernel)", name)
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


def source_digest(path: str) -> str:
    """sha256 of a kernel source file's code (comments and whitespace do not count): counter
    readings are void once the kernels' code changes."""
    return hashlib.sha256(_code_only(open(path).read()).encode()).hexdigest()


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
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
    a = ap.parse_args()
    if a.cmd == "stats":
        with open(a.out, "w") as f:
            f.write(stats_summary(a.csv, a.command))
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
