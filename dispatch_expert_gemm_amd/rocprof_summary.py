"""Summarise rocprofv3 CSV output into short text for the profiles/ folder.

    python -m dispatch_expert_gemm_amd.rocprof_summary stats <kernel_stats.csv> [--cmd "..."]
    python -m dispatch_expert_gemm_amd.rocprof_summary pmc <counter_collection.csv> [--cmd "..."]

`stats` prints per-kernel calls and average / total duration from a --kernel-trace --stats run.
`pmc` prints, per kernel, the mean per-dispatch value of every counter (summed over the
counter's hardware instances) from a --pmc run.
"""
from __future__ import annotations

import argparse
import collections
import csv
import sys


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        calls = int(r["Calls"])
        avg = float(r["AverageNs"]) / 1e3
        tot = float(r["TotalDurationNs"]) / 1e3
        out.append(f"| `{name[:90]}` | {calls} | {avg:.2f} | {tot:.1f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out)


def pmc(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in rows:
        k = r["Kernel_Name"]
        per[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
    out = ["| kernel | dispatches | counter | mean per dispatch |", "|---|---:|---|---:|"]
    for k, c in per.items():
        n = len(disp[k])
        for name, v in sorted(c.items()):
            out.append(f"| `{k[:90]}` | {n} | {name} | {v / n:.1f} |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["stats", "pmc"])
    ap.add_argument("csv")
    ap.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    text = stats(a.csv) if a.kind == "stats" else pmc(a.csv)
    if a.cmd:
        print(f"Command: `{a.cmd}`\n")
    print(text)


if __name__ == "__main__":
    sys.exit(main())
