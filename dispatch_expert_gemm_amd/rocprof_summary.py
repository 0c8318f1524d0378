"""Summarise rocprofv3 CSV output into short text for the profiles/ folder.

    python -m dispatch_expert_gemm_amd.rocprof_summary stats <kernel_stats.csv> [--cmd "..."]
    python -m dispatch_expert_gemm_amd.rocprof_summary pmc <counter_collection.csv> [--cmd "..."]
    python -m dispatch_expert_gemm_amd.rocprof_summary traffic <FETCH_SIZE.csv> <WRITE_SIZE.csv>
        --kernel PREFIX --workload NAME --source FILE --copy-mib M [--cmd "..."]

`stats` prints per-kernel calls and average / total duration from a --kernel-trace --stats run.
`pmc` prints, per kernel, the mean per-dispatch value of every counter (summed over the
counter's hardware instances) from a --pmc run.
`traffic` turns a FETCH_SIZE run and a WRITE_SIZE run (each with one device-to-device copy of M MiB
as a kernel of known traffic) into HBM bytes per launch of the kernels named PREFIX...: each
counter is scaled by what it reads for the copy, and the result ends with one `traffic-record:`
line (JSON) that the benchmark reads, tied to the SHA-256 of the kernel source's code (comments
and whitespace removed).
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


def _per_kernel(path: str, counter: str):
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        tot[r["Kernel_Name"]] += float(r["Counter_Value"])
        disp[r["Kernel_Name"]].add(r["Dispatch_Id"])
    return tot, disp


def _first_dispatch(path: str, counter: str, name_part: str) -> float:
    """Counter value of the earliest dispatch whose kernel name contains name_part (summed over
    the rows of that dispatch)."""
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{counter}: no dispatch of {name_part} in {path}")
    return per[min(per)]


def code_hash(path: str) -> str:
    """SHA-256 of a C++/HIP source with its // comments and all whitespace removed, so that a
    counter record stays tied to the code and not to its comments."""
    import hashlib
    import re
    text = open(path).read()
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()


def traffic(fetch_csv: str, write_csv: str, kernel: str, workload: str, source: str,
            copy_mib: int) -> str:
    import json
    import os
    copy_kib = copy_mib * 1024.0
    out = []
    rec = {"workload": workload, "kernel_prefix": kernel, "source": os.path.basename(source),
           "source_code_sha256": code_hash(source)}
    per_launch = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        tot, disp = _per_kernel(path, name)
        # the calibration copy is the program's first device-to-device copy (later copies,
        # such as a bandwidth reference, are not counted)
        copy = _first_dispatch(path, name, "copyBuffer")
        scale = copy_kib / copy
        ks = [k for k in tot if k.removeprefix("void ").startswith(kernel)]
        if len(ks) != 1:
            raise SystemExit(f"{name}: expected one kernel matching {kernel}, found {ks}")
        raw = tot[ks[0]] / len(disp[ks[0]])
        per_launch += raw * scale * 1024.0
        rec[name.lower() + "_kib_raw"] = round(raw, 1)
        rec[name.lower() + "_scale"] = round(scale, 4)
        out.append(f"| {name} | `{ks[0][:70]}` | {len(disp[ks[0]])} | {raw:.1f} | "
                   f"{copy:.0f} KiB for the {copy_mib} MiB copy | {scale:.4f} | "
                   f"{raw * scale / 1024:.1f} MiB |")
    rec["bytes_per_launch"] = int(per_launch)
    head = ["| counter | kernel | dispatches | KiB per dispatch (raw) | copy calibration | scale | "
            "scaled per launch |", "|---|---|---:|---:|---|---:|---:|"]
    return "\n".join(head + out + ["", f"HBM bytes per launch: {per_launch / 1e9:.3f} GB", "",
                                      "traffic-record: " + json.dumps(rec, sort_keys=True)])


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["stats", "pmc", "traffic"])
    ap.add_argument("csv")
    ap.add_argument("csv2", nargs="?")
    ap.add_argument("--cmd", default=[], action="append")
    ap.add_argument("--kernel", default="")
    ap.add_argument("--workload", default="")
    ap.add_argument("--source", default="")
    ap.add_argument("--copy-mib", type=int, default=1024)
    a = ap.parse_args(argv)
    if a.kind == "stats":
        text = stats(a.csv)
    elif a.kind == "pmc":
        text = pmc(a.csv)
    else:
        text = traffic(a.csv, a.csv2, a.kernel, a.workload, a.source, a.copy_mib)
    for c in a.cmd:
        if c:
            print(f"Command: `{c}`\n")
    print(text)


if __name__ == "__main__":
    sys.exit(main())
