"""Turn rocprofv3 output of bench.py into a short text summary.

The summary is what profiles/*.md hold: per-kernel average durations from a
kernel trace, and the bytes each dispatch moves between the L2 caches and
memory from FETCH_SIZE / WRITE_SIZE counter passes, each scaled by what the
same counter reads for a plain device copy of known size (bench.py
--copy-calibration).  FETCH_SIZE counts L2 misses: bytes served by HBM or by
the last-level (Infinity) cache in front of it, which no counter of this
tool tells apart.  Averages cover the timed steps only: bench.py runs W
warm-up steps and then K timed steps with the same kernels, so the last
K / (W + K) of each kernel's dispatches are the timed ones.  The summary also
records a hash of the code of the HIP sources behind the profiled kernels
(comments and whitespace left out), so bench.py can tell whether the measured
traffic still describes the kernels it runs.

Expected layout of the rocprofv3 output directory (one `-d` per pass, `-o run`
and `-f csv`):
    trace/       --kernel-trace --stats           (bench.py)
    fetch/       --pmc FETCH_SIZE                 (bench.py)
    write/       --pmc WRITE_SIZE                 (bench.py)
    copy_fetch/  --pmc FETCH_SIZE                 (bench.py --copy-calibration MIB)
    copy_write/  --pmc WRITE_SIZE                 (bench.py --copy-calibration MIB)
plus copy_fetch.json, the calibration run's stdout, and trace_bench.json, the
traced bench run's stdout (its steps and warmup pick the timed dispatches).

Usage: python -m yoco_shared_kv_gather_amd.profiling OUTDIR --workload NAME --stem X --command "..." > profiles/X.md
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import statistics
from typing import Dict, List, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
ROOT = os.path.dirname(PKG_DIR)
PROFILES = os.path.join(ROOT, "profiles")


# the sources a profile's kernels are built from, by profile name prefix
FAMILIES = {
    "cross_attn_": ["cross_attn*", "kv_append.hip", "gather_last.hip", "yoco_internal.h"],
    "gated_retention_": ["retention.hip", "yoco_internal.h"],
}


def family_sources(stem: Optional[str]) -> List[str]:
    """The HIP sources behind the kernels of profile `stem` (every source when
    the stem names no family), plus the public header."""
    patterns = ["*"]
    for prefix, pats in FAMILIES.items():
        if stem is not None and stem.startswith(prefix):
            patterns = pats
    files = sorted({f for pat in patterns for f in glob.glob(os.path.join(CSRC, pat))})
    return files + [os.path.join(ROOT, "include", "yoco.h")]


def code_only(text: str) -> str:
    """C/C++ source without its comments, every run of whitespace as one
    space: what the compiler sees, so that editing a comment leaves the hash
    alone.  String and character literals are kept whole (a // inside one is
    not a comment)."""
    out = []
    i, n = 0, len(text)
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


def source_hash(stem: Optional[str] = None) -> str:
    """sha256 over the code (comments and whitespace left out) of profile
    `stem`'s kernel sources and the public header, in name order (all
    sources without a stem)."""
    h = hashlib.sha256()
    for path in family_sources(stem):
        h.update(os.path.basename(path).encode())
        with open(path, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("yoco_attn::", "")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, c in enumerate(name):
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == "(" and depth == 0:
            return name[:i]
    return name


def _timed(values: List[float], steps: int, warmup: int) -> List[float]:
    """The timed steps' share of one kernel's dispatches (in dispatch order):
    the last steps / (warmup + steps) of them, when the count divides evenly
    (else all of them)."""
    total = steps + warmup
    if steps <= 0 or total <= 0 or len(values) % total != 0:
        return values
    per_step = len(values) // total
    return values[warmup * per_step:]


def _counters(path: str, steps: int = 0, warmup: int = 0) -> Dict[str, List[float]]:
    rows: Dict[str, List[tuple]] = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            rows[row["Kernel_Name"]].append((int(row.get("Dispatch_Id") or 0), float(row["Counter_Value"])))
    return {name: _timed([v for _, v in sorted(vals)], steps, warmup) for name, vals in rows.items()}


def _durations(path: str, steps: int, warmup: int) -> Dict[str, List[float]]:
    """Per-dispatch durations (ns) of each kernel from the kernel trace, timed
    steps only."""
    rows: Dict[str, List[tuple]] = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            rows[row["Kernel_Name"]].append((int(row["Start_Timestamp"]),
                                             int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
    return {name: _timed([d for _, d in sorted(vals)], steps, warmup) for name, vals in rows.items()}


def _calibration(out: str, sub: str) -> float:
    """Bytes per counter unit, from the plain copy of known size."""
    copy_bytes = json.load(open(os.path.join(out, "copy_fetch.json")))["copy_calibration_bytes"]
    counts = _counters(os.path.join(out, sub, "run_counter_collection.csv"))
    # the copy is the kernel with the largest reading in the calibration run
    best = max(statistics.median(v) for v in counts.values())
    return copy_bytes / best


def summarize(out: str, workload: str, command: str, top: int = 10, stem: Optional[str] = None) -> str:
    bench = json.load(open(os.path.join(out, "trace_bench.json")))
    steps, warmup = int(bench.get("steps", 0)), int(bench.get("warmup", 0))
    stats = list(csv.DictReader(open(os.path.join(out, "trace", "run_kernel_stats.csv"))))
    durations = _durations(os.path.join(out, "trace", "run_kernel_trace.csv"), steps, warmup)
    fetch = _counters(os.path.join(out, "fetch", "run_counter_collection.csv"), steps, warmup)
    write = _counters(os.path.join(out, "write", "run_counter_collection.csv"), steps, warmup)
    f_scale = _calibration(out, "copy_fetch")
    w_scale = _calibration(out, "copy_write")
    lines = [
        f"# rocprofv3 summary: {workload}",
        "",
        f"source_hash: {source_hash(stem)}",
        f"sources: {', '.join(os.path.relpath(f, ROOT) for f in family_sources(stem))}",
        f"workload: {workload}",
        f"counter_scale_fetch_bytes_per_unit: {f_scale:.4f}",
        f"counter_scale_write_bytes_per_unit: {w_scale:.4f}",
        "",
        "Commands (run from the repository root on the GPU machine):",
        "",
        "```",
        command.strip(),
        "```",
        "",
        f"bench.py line of the traced run: ms_per_step {bench['ms_per_step']}, value {bench['value']} {bench['unit']}, "
        f"roofline achieved {bench['roofline']['achieved']} {bench['roofline']['unit']} (event-timed)",
        "",
        f"Kernels of this library only (input generation and cache flushing omitted).  Times and bytes are "
        f"averages over the {steps} timed steps' dispatches ({warmup} warm-up steps left out).  'L2-miss read' is "
        f"FETCH_SIZE and 'L2 write-back' WRITE_SIZE, scaled to bytes by the plain copy: traffic between the L2s and "
        f"memory, where a read may be served by HBM or by the last-level (Infinity) cache.",
        "",
        "| kernel | timed calls | avg us | L2-miss read MB/dispatch | L2 write-back MB/dispatch |",
        "|---|---:|---:|---:|---:|",
    ]
    records = {}
    ours = [row for row in stats
            if not short_name(row["Name"]).startswith(("at::", "__amd", "c10::", "rocprim::", "hipcub::"))
            and "at::native" not in row["Name"]]
    for row in ours[:top]:
        name = row["Name"]
        fr = statistics.mean(fetch[name]) * f_scale if fetch.get(name) else None
        wr = statistics.mean(write[name]) * w_scale if write.get(name) else None
        timed = durations.get(name) or []
        avg_us = statistics.mean(timed) / 1e3 if timed else float(row["AverageNs"]) / 1e3
        records[short_name(name)] = (avg_us, fr, wr)
        lines.append(f"| {short_name(name)} | {len(timed)} | {avg_us:.2f} | "
                     f"{'' if fr is None else f'{fr / 1e6:.2f}'} | {'' if wr is None else f'{wr / 1e6:.2f}'} |")
    lines.append("")
    for name, (avg_us, fr, wr) in records.items():
        if fr is not None and wr is not None:
            lines.append(f"kernel_bytes: {name} | {avg_us:.3f} | {fr:.0f} | {wr:.0f}")
    return "\n".join(lines) + "\n"


def per_position(out: str, kernel: str) -> List[str]:
    """Average duration of `kernel` by its position within a step (the k-th
    dispatch of the kernel in each timed step): for the cross layers, layer k.
    Shows what a layer gains from the last-level cache holding blocks the
    previous layer read (the first layer of a step starts cold)."""
    bench = json.load(open(os.path.join(out, "trace_bench.json")))
    steps, warmup = int(bench.get("steps", 0)), int(bench.get("warmup", 0))
    durations = _durations(os.path.join(out, "trace", "run_kernel_trace.csv"), steps, warmup)
    name = next((n for n in durations if short_name(n) == kernel), None)
    if name is None or steps <= 0 or len(durations[name]) % steps != 0:
        return []
    per_step = len(durations[name]) // steps
    lines = [f"Per-layer average of {kernel} over the {steps} timed steps (layer order "
             f"{'alternating' if bench['config'].get('alternating_layer_order', True) else 'the same every layer'}):",
             "", "| layer | avg us |", "|---:|---:|"]
    for k in range(per_step):
        vals = durations[name][k::per_step]
        lines.append(f"| {k} | {statistics.mean(vals) / 1e3:.2f} |")
    return lines + [""]


def extra_counters(out: str, sub: str, kernels: List[str]) -> List[str]:
    """Timed-step averages per dispatch of every counter in pass `sub` (raw
    counter units, summed over the GPU's instances), for `kernels`."""
    bench = json.load(open(os.path.join(out, "trace_bench.json")))
    steps, warmup = int(bench.get("steps", 0)), int(bench.get("warmup", 0))
    rows: Dict[tuple, List[tuple]] = collections.defaultdict(list)
    with open(os.path.join(out, sub, "run_counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if short_name(row["Kernel_Name"]) in kernels:
                rows[(short_name(row["Kernel_Name"]), row["Counter_Name"])].append(
                    (int(row.get("Dispatch_Id") or 0), float(row["Counter_Value"])))
    lines = [f"Counter pass `{sub}` (timed-step average per dispatch):", "", "| kernel | counter | value |",
             "|---|---|---:|"]
    for (kname, counter), vals in sorted(rows.items()):
        timed = _timed([v for _, v in sorted(vals)], steps, warmup)
        lines.append(f"| {kname} | {counter} | {statistics.mean(timed):.6g} |")
    return lines + [""]


def measured_traffic(stem: str, kernels: List[str]) -> Optional[dict]:
    """L2-miss bytes per dispatch and average kernel time summed over `kernels`,
    from the committed profile profiles/<stem>.md -- or None if there is none
    or the sources changed since."""
    path = os.path.join(PROFILES, f"{stem}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_hash: (\S+)", text, re.M)
    if not m or m.group(1) != source_hash(stem):
        return None
    total_r = total_w = total_us = 0.0
    found = 0
    for line in text.splitlines():
        if line.startswith("kernel_bytes: "):
            name, us, r, w = [f.strip() for f in line[len("kernel_bytes: "):].split("|")]
            if name in kernels:
                total_r += float(r)
                total_w += float(w)
                total_us += float(us)
                found += 1
    if found != len(kernels):
        return None
    return {"read_bytes": total_r, "write_bytes": total_w, "kernel_us": total_us,
            "profile": os.path.relpath(path, ROOT)}


def main():
    p = argparse.ArgumentParser(description="summarize rocprofv3 output of bench.py")
    p.add_argument("out")
    p.add_argument("--workload", required=True)
    p.add_argument("--command", required=True, help="the commands that produced OUT (recorded in the summary)")
    p.add_argument("--stem", default=None, help="profile file name without .md (picks the sources hashed)")
    p.add_argument("--per-position", default=None, help="kernel (short name) to break down by layer")
    p.add_argument("--extra", action="append", default=[], metavar="SUBDIR",
                   help="extra counter pass under OUT to tabulate for the --kernels")
    p.add_argument("--kernels", action="append", default=[], help="short kernel names for --extra")
    args = p.parse_args()
    text = summarize(args.out, args.workload, args.command, stem=args.stem)
    extra = []
    if args.per_position:
        extra += per_position(args.out, args.per_position)
    for sub in args.extra:
        extra += extra_counters(args.out, sub, args.kernels)
    print(text + ("\n" + "\n".join(extra) if extra else ""), end="")


if __name__ == "__main__":
    main()
