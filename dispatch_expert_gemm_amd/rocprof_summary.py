"""Summarise rocprofv3 CSV output into short text for the profiles/ folder.

    python -m dispatch_expert_gemm_amd.rocprof_summary stats <kernel_stats.csv> [<kernel_trace.csv>
        --last N] [--cmd "..."]
    python -m dispatch_expert_gemm_amd.rocprof_summary pmc <counter_collection.csv> [--cmd "..."]
    python -m dispatch_expert_gemm_amd.rocprof_summary busy <counter_collection.csv> [--cus 256]
        [--xcds 8] [--last N] [--cmd "..."]
    python -m dispatch_expert_gemm_amd.rocprof_summary traffic <FETCH_SIZE.csv> <WRITE_SIZE.csv>
        --kernel PREFIX --workload NAME --source FILE --copy-mib M [--last N] [--cmd "..."]
    python -m dispatch_expert_gemm_amd.rocprof_summary timeline <kernel_trace.csv>
        --kernel PREFIX --step N [--before-us T] [--cmd "..."]

`stats` prints per-kernel calls and average / total duration from a --kernel-trace --stats run;
given the run's kernel trace and --last N it adds each kernel's mean over its last N dispatches
(the launches of a program's final timed loop).
`pmc` prints, per kernel, the mean per-dispatch value of every counter (summed over the
counter's hardware instances) from a --pmc run.
`busy` reads a --pmc run holding GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES (SQ_BUSY_CYCLES
and SQ_WAVES optional) and prints, per kernel, the mean duration, the clock it ran at (the
graphics-busy cycles of one XCD over the duration, for kernels of 100 us or more; the counter
as reported sums the XCDs) and
the fraction of SIMD cycles with the matrix core busy (MFMA busy cycles over busy cycles x CUs x
4 SIMDs), over all dispatches or each kernel's last N.
`traffic` turns a FETCH_SIZE run and a WRITE_SIZE run (each with one device-to-device copy of M MiB
as a kernel of known traffic) into HBM bytes per launch of the kernels named PREFIX... (over
their last N dispatches with --last N): each
counter is scaled by what it reads for the copy, and the result ends with one `traffic-record:`
line (JSON) that the benchmark reads, tied to the SHA-256 of the kernel source's code (comments
and whitespace removed).
`timeline` lists the dispatches of one step of a kernel trace: the step runs from the N-th
dispatch (0-based, by start time) of the kernel named PREFIX... to the next one, and the list also
holds dispatches that start up to T us before it (work another queue began first); times are in
us from the step's first dispatch, with each dispatch's hardware queue.
"""
from __future__ import annotations

import argparse
import collections
import csv
import sys


def last_dispatches(trace_csv: str, n: int) -> dict:
    """Mean duration in us of each kernel's last n dispatches (by start time) in a kernel trace."""
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = {}
    for k, v in per.items():
        v.sort()
        tail = v[-n:]
        out[k] = sum(e - b for b, e in tail) / len(tail) / 1e3
    return out


def timeline(trace_csv: str, kernel: str, step: int, before_us: float = 0.0) -> str:
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    anchors = [i for i, r in enumerate(rows) if r["Kernel_Name"].startswith(kernel)]
    if step + 1 >= len(anchors):
        raise ValueError(f"{len(anchors)} dispatches of {kernel}: no step {step}")
    t0 = int(rows[anchors[step]]["Start_Timestamp"])
    t1 = int(rows[anchors[step + 1]]["Start_Timestamp"])
    sel = [r for r in rows if t0 - before_us * 1e3 <= int(r["Start_Timestamp"]) < t1]
    out = ["| queue | kernel | start us | end us | us |", "|---:|---|---:|---:|---:|"]
    for r in sel:
        b = (int(r["Start_Timestamp"]) - t0) / 1e3
        e = (int(r["End_Timestamp"]) - t0) / 1e3
        name = r["Kernel_Name"].split("(")[0][:60]
        out.append(f"| {r['Queue_Id']} | `{name}` | {b:.1f} | {e:.1f} | {e - b:.1f} |")
    last_end = max((int(r["End_Timestamp"]) for r in sel), default=t0)
    out.append("")
    out.append(f"step {step}: {(last_end - t0) / 1e3:.1f} us from the first {kernel} dispatch to "
               f"the last end; next step starts at {(t1 - t0) / 1e3:.1f} us")
    return "\n".join(out)


def stats(path: str, trace_csv: str | None = None, last: int = 0) -> str:
    rows = list(csv.DictReader(open(path)))
    tail = last_dispatches(trace_csv, last) if trace_csv and last > 0 else None
    head = "| kernel | calls | avg us | total us | % |"
    rule = "|---|---:|---:|---:|---:|"
    if tail is not None:
        head += f" avg us, last {last} |"
        rule += "---:|"
    out = [head, rule]
    for r in rows:
        name = r["Name"]
        calls = int(r["Calls"])
        avg = float(r["AverageNs"]) / 1e3
        tot = float(r["TotalDurationNs"]) / 1e3
        line = f"| `{name[:90]}` | {calls} | {avg:.2f} | {tot:.1f} | {float(r['Percentage']):.2f} |"
        if tail is not None:
            line += f" {tail[name]:.2f} |" if name in tail else " |"
        out.append(line)
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


def busy(path: str, cus: int, xcds: int, last: int = 0) -> str:
    rows = list(csv.DictReader(open(path)))
    keep = None
    if last > 0:        # each kernel's last `last` dispatches by dispatch id
        ids = collections.defaultdict(set)
        for r in rows:
            ids[r["Kernel_Name"]].add(int(r["Dispatch_Id"]))
        keep = {(k, d) for k, v in ids.items() for d in sorted(v)[-last:]}
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = collections.defaultdict(dict)
    for r in rows:
        k, d = r["Kernel_Name"], int(r["Dispatch_Id"])
        if keep is not None and (k, d) not in keep:
            continue
        per[k][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[k][d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = ["| kernel | dispatches | mean us | clock GHz | MFMA busy | SQ busy / XCD cycle | "
           "waves per dispatch |", "|---|---:|---:|---:|---:|---:|---:|"]
    for k, c in per.items():
        if "GRBM_GUI_ACTIVE" not in c or "SQ_VALU_MFMA_BUSY_CYCLES" not in c:
            continue
        n = len(dur[k])
        ns = sum(dur[k].values()) / n
        gui = c["GRBM_GUI_ACTIVE"] / n / xcds          # cycles of one XCD per dispatch
        clock = gui / ns if ns > 0 else 0.0
        mfma = c["SQ_VALU_MFMA_BUSY_CYCLES"] / n / (gui * cus * 4) if gui else 0.0
        sq = c.get("SQ_BUSY_CYCLES", 0.0) / n / gui if gui else 0.0
        waves = c.get("SQ_WAVES", 0.0) / n
        # the busy counter also runs for some microseconds around the kernel, so the clock is
        # shown only for kernels long enough for that to vanish
        shown = f"{clock:.3f}" if ns >= 100e3 else "-"
        out.append(f"| `{k[:80]}` | {n} | {ns / 1e3:.1f} | {shown} | {100 * mfma:.1f}% | "
                   f"{sq:.2f} | {waves:.0f} |")
    return "\n".join(out)


def _per_kernel(path: str, counter: str, last: int = 0):
    """Per kernel: the counter summed over its dispatches (only its last `last` dispatches by
    dispatch id when last > 0) and the set of dispatches counted."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per[r["Kernel_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    tot, disp = {}, {}
    for k, v in per.items():
        ids = sorted(v)[-last:] if last > 0 else sorted(v)
        tot[k] = sum(v[i] for i in ids)
        disp[k] = set(ids)
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
            copy_mib: int, last: int = 0) -> str:
    import json
    import os
    copy_kib = copy_mib * 1024.0
    out = []
    rec = {"workload": workload, "kernel_prefix": kernel, "source": os.path.basename(source),
           "source_code_sha256": code_hash(source)}
    per_launch = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        tot, disp = _per_kernel(path, name, last)
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
    ap.add_argument("kind", choices=["stats", "pmc", "busy", "traffic", "timeline"])
    ap.add_argument("csv")
    ap.add_argument("csv2", nargs="?")
    ap.add_argument("--cmd", default=[], action="append")
    ap.add_argument("--kernel", default="")
    ap.add_argument("--workload", default="")
    ap.add_argument("--source", default="")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--last", type=int, default=0)
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--xcds", type=int, default=8)
    ap.add_argument("--step", type=int, default=0)
    ap.add_argument("--before-us", type=float, default=0.0)
    a = ap.parse_args(argv)
    if a.kind == "stats":
        text = stats(a.csv, a.csv2, a.last)
    elif a.kind == "pmc":
        text = pmc(a.csv)
    elif a.kind == "busy":
        text = busy(a.csv, a.cus, a.xcds, a.last)
    elif a.kind == "timeline":
        text = timeline(a.csv, a.kernel, a.step, a.before_us)
    else:
        text = traffic(a.csv, a.csv2, a.kernel, a.workload, a.source, a.copy_mib, a.last)
    for c in a.cmd:
        if c:
            print(f"Command: `{c}`\n")
    print(text)


if __name__ == "__main__":
    sys.exit(main())
