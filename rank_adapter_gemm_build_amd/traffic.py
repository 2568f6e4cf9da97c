"""HBM traffic per launch from rocprofv3 counter runs (diagnostics, not the hot path).

Two runs of the same bench command with ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``
give per-dispatch counter values in KiB.  The same bench run also launches a plain
copy of 512 MiB, whose true traffic is known (512 MiB read, 512 MiB written); the
ratio of that to the copy's counter values is the calibration factor applied to the
LoRA kernels' values.  The result is merged into ``profiles/traffic.json`` under the
workload's name, tagged with the digest of the kernel sources it was measured on,
so a later change to the kernels makes the entry stale (bench.py then reports
``traffic: null``).

Usage:
    python -m rank_adapter_gemm_build_amd.traffic WORKLOAD_NAME FETCH_CSV WRITE_CSV [COMMAND]
    python -m rank_adapter_gemm_build_amd.traffic --stats STATS_CSV OUT_MD TITLE COMMAND
(the second form writes a short markdown summary of a rocprofv3 --stats table)
"""
from __future__ import annotations

import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
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
    m = re.search(r"rax::(shrink|expand|routing|finish_u)_kernel", name)
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


def main(argv):
    if len(argv) >= 2 and argv[1] == "--stats":
        stats_markdown(argv[2], argv[3], argv[4], argv[5])
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
