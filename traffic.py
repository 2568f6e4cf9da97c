"""Summaries of rocprofv3 runs of bench.py for profiles/ (measurement tooling, not part
of the library).

HBM traffic per launch from rocprofv3 counter runs:

Two runs of the same bench command with ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``
give per-dispatch counter values in KiB.  The same bench run also launches a plain
copy of 512 MiB, whose true traffic is known (512 MiB read, 512 MiB written); the
ratio of that to the copy's counter values is the calibration factor applied to the
LoRA kernels' values.  The result is merged into ``profiles/traffic.json`` under the
workload's name, tagged with the digest of the kernel sources it was measured on,
so a later change to the kernels makes the entry stale (bench.py then reports
``traffic: null``).

Usage:
    python traffic.py WORKLOAD_NAME FETCH_CSV WRITE_CSV [COMMAND]
    python traffic.py --stats STATS_CSV OUT_MD TITLE COMMAND
    python traffic.py --overlap KERNEL_TRACE_CSV OUT_MD COMMAND
(the second form writes a short markdown summary of a rocprofv3 --stats table; the
third the per-step timeline of bench.py --only-overlap from a --kernel-trace run)
"""
from __future__ import annotations

import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 512 * 2 ** 20


def _per_dispatch(path: str, counter: str):
    """[(kernel name, grid size, value in KiB)] in dispatch order."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            grid = int(r.get("Grid_Size", r.get("Grid_Size_X", "0")) or 0)
            rows.append((r["Kernel_Name"], grid, float(r["Counter_Value"])))
    return rows


def _family(name: str):
    m = re.search(r"rax::(shrink|expand|routing|finish_u)(?:_slot)?(?:_group)?_kernel", name)
    return {"routing": "routing", "finish_u": "finish_u"}.get(m.group(1), m.group(1)) if m else None


def _copy_values(rows):
    # the 512 MiB copy: the dispatches with the largest counter values outside the library
    vals = sorted((v for n, g, v in rows if _family(n) is None and "copy" in n.lower()), reverse=True)
    big = [v for v in vals if v > 0.5 * vals[0]] if vals else []
    return sum(big) / len(big) if big else None


def summarize(fetch_csv: str, write_csv: str):
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _per_dispatch(path, counter)
        copy_kib = _copy_values(rows)
        if not copy_kib:
            raise SystemExit(f"no copy dispatch found in {path}")
        factor = COPY_BYTES / (copy_kib * 1024.0)
        fam = {}
        for n, g, v in rows:
            k = _family(n)
            if k in ("shrink", "expand"):
                fam.setdefault(k, []).append(v)
        for k, vs in fam.items():
            e = out.setdefault(k, {})
            e[counter.lower() + "_bytes_per_launch"] = sum(vs) / len(vs) * 1024.0 * factor
            e[counter.lower() + "_factor"] = factor
            e["dispatches"] = len(vs)
    for k, e in out.items():
        e["bytes_per_launch"] = int(e.get("fetch_size_bytes_per_launch", 0) + e.get("write_size_bytes_per_launch", 0))
    return out


def stats_markdown(stats_csv: str, out_md: str, title: str, command: str):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (from the repository root; rocprofv3 writes the CSV named below):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = re.sub(r"\(.*", "", name)
        lines.append(f"| `{short[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _trace_rows(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            kind = ("gemm" if name.startswith("Cijk") or "gemm" in name.lower() else
                    "shrink" if re.search(r"rax::shrink(_slot)?(_group)?_kernel", name) else
                    "expand" if re.search(r"rax::expand(_slot)?(_group)?_kernel", name) else "other")
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kind, r.get("Queue_Id", "?")))
    rows.sort()
    return rows


def overlap_markdown(trace_csv: str, out_md: str, command: str, gap_ns: int = 1_000_000):
    """The forms of bench.py --only-overlap (base GEMM alone; GEMM then LoRA on one stream;
    GEMM and LoRA on two streams joined by an event, steps chained; the same with
    independent steps; then the GEMM alone, the serial step and the forked step captured
    in HIP graphs), separated by idle gaps of more than 1 ms: per form and step,
    when the GEMM, the shrink and the expand run, and the idle time between the GEMM's
    end and the expand's start (the event wait)."""
    rows = [r for r in _trace_rows(trace_csv) if r[2] != "other"]
    phases, cur = [], []
    for r in rows:
        if cur and r[0] - max(c[1] for c in cur) > gap_ns:
            phases.append(cur)
            cur = []
        cur.append(r)
    if cur:
        phases.append(cur)
    # the forms are the first four stretches with base GEMMs in them (earlier stretches are
    # the set-up and the warm-up steps of the LoRA step alone)
    phases = [ph for ph in phases if sum(1 for r in ph if r[2] == "gemm") >= 5]
    # eager forms, then per graph three stretches: its warm-up steps (eager, on a side
    # stream), its first replay and the timed replays
    phases = phases[:4] + phases[6::3][:3]
    names = ["base GEMM alone", "GEMM then LoRA, one stream", "GEMM beside LoRA, joined, chained steps",
             "GEMM beside LoRA, joined, independent steps", "HIP graph: base GEMM alone",
             "HIP graph: GEMM then LoRA, one stream", "HIP graph: GEMM on a forked stream, LoRA joined to it"]
    lines = [f"# Base-GEMM overlap timeline, decode workload (64 tokens, 8 slots, k = d = 4096, r = 16)", "",
             "Command (from the repository root; rocprofv3 writes the kernel trace named below):", "", "```",
             command, "```", "",
             "Per form: the last steps' mean durations and gaps from the kernel trace (start and end stamps of",
             "each dispatch, in microseconds; the tracer itself lengthens every gap between kernels). 'us per",
             "step' is the time from one base GEMM's start to the next; 'wait' is the time from a GEMM's end to",
             "the start of the expand of the same step (on one stream the shrink runs in between); 'shrink",
             "beside GEMM' is the part of the shrink that runs while the GEMM runs.", "",
             "| form | steps | us per step | GEMM us | shrink us | expand us | wait us | shrink beside GEMM us | queues |",
             "|---|---|---|---|---|---|---|---|---|"]
    for name, ph in zip(names, phases):
        gem = [r for r in ph if r[2] == "gemm"]
        shr = [r for r in ph if r[2] == "shrink"]
        exp = [r for r in ph if r[2] == "expand"]
        n = len(gem)
        if n < 2:
            continue
        k = max(1, min(n, len(exp), 20) if exp else min(n, 20))
        gem, shr, exp = gem[-k:], shr[-k:], exp[-k:]
        starts = [g[0] for g in gem]
        per_step = (starts[-1] - starts[0]) / (len(starts) - 1) / 1e3   # GEMM start to the next GEMM start
        dur = lambda rs: sum(r[1] - r[0] for r in rs) / len(rs) / 1e3 if rs else 0.0
        waits, beside = [], []
        for g, e in zip(gem, exp):
            waits.append(max(0, e[0] - g[1]) / 1e3)
        for g, s in zip(gem, shr):
            beside.append(max(0, min(g[1], s[1]) - max(g[0], s[0])) / 1e3)
        mean = lambda v: sum(v) / len(v) if v else 0.0
        queues = sorted({r[3] for r in ph})
        lines.append(f"| {name} | {k} | {per_step:.1f} | {dur(gem):.1f} | {dur(shr):.1f} | {dur(exp):.1f} | "
                     f"{mean(waits):.1f} | {mean(beside):.1f} | {len(queues)} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv):
    if len(argv) >= 2 and argv[1] == "--stats":
        stats_markdown(argv[2], argv[3], argv[4], argv[5])
        return 0
    if len(argv) >= 2 and argv[1] == "--overlap":
        overlap_markdown(argv[2], argv[3], argv[4])
        return 0
    if len(argv) < 4:
        print(__doc__)
        return 2
    sys.path.insert(0, ROOT)
    from bench import source_digest  # the digest bench.py compares against

    name, fetch_csv, write_csv = argv[1], argv[2], argv[3]
    command = argv[4] if len(argv) > 4 else ""
    res = summarize(fetch_csv, write_csv)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            allv = json.load(f)
    except (OSError, ValueError):
        allv = {}
    dig = source_digest()
    for k, e in res.items():
        e["source_digest"] = dig
        e["command"] = command
    allv[name] = res
    with open(path, "w") as f:
        json.dump(allv, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
