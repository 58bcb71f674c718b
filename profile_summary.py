#!/usr/bin/env python3
"""Turn rocprofv3 CSV output of bench.py runs into the short text summaries
kept under profiles/ and the per-launch HBM traffic record bench.py reads.

  python profile_summary.py trace   --dir D --kernel REGEX --steps N --out F --command CMD
      kernel-trace statistics of every kernel in D, plus the mean duration of
      the last N dispatches of the kernel matching REGEX (bench.py's timed
      launches) -- the figure to compare with bench.py's HIP-event timing.

  python profile_summary.py counters --dir D [--dir D2] --kernel REGEX --title T --out F
                                    --command CMD [--command CMD ...] [--source-key KEY]
      median per-dispatch value of every counter collected for the kernel,
      plus the MFMA utilisation and stall fractions derived from them.

  python profile_summary.py traffic --fetch D1 --write D2 --calib-fetch D3 --calib-write D4
                                    --kernel REGEX --name KERNEL --workload W --out-json J
                                    --out-txt F --command CMD [--command CMD ...]
      FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel, each scaled
      by the ratio of known bytes to the same counter's reading for a plain
      elementwise copy of 512 MiB (bench.py --calibrate-copy).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def _rows(d: str, suffix: str):
    """Rows of every rocprofv3 CSV with this suffix under d (one file per
    profiled process), each tagged with its file so dispatch ids of different
    processes stay apart."""
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {d}")
    out = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                r["_file"] = fn
                out.append(r)
    return out


def trace(a):
    rows = _rows(a.dir, "kernel_trace.csv")
    by = {}
    for r in rows:
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), dur))
    lines = [f"# rocprofv3 kernel trace: {a.title}", "", "Command (from the repository root):", "",
             f"    {a.command}", "",
             "| kernel | dispatches | mean us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    pat = re.compile(a.kernel)
    timed = []
    others = 0
    for name, v in sorted(by.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        if not pat.search(name):
            others += 1
            continue
        durs = [d / 1e3 for _, d in v]
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {len(durs)} | {statistics.mean(durs):.2f} | "
                     f"{statistics.median(durs):.2f} | {min(durs):.2f} | {max(durs):.2f} |")
        last = [d / 1e3 for _, d in sorted(v)[-a.steps:]]
        timed.append((short, len(last), statistics.mean(last), statistics.median(last)))
    if not timed:
        sys.exit(f"no kernel matches {a.kernel}")
    lines += ["", f"({others} other kernels of the traced process -- input set-up, copies, "
              "other bench legs -- are not listed.)"]
    lines += ["", f"Timed launches: the last {timed[0][1]} dispatches of each kernel matching "
              f"`{a.kernel}` (the ones bench.py times after its warm-up):", ""]
    lines += [f"- `{n}`: mean {mn:.2f} us, median {md:.2f} us" for n, _, mn, md in timed]
    if len(timed) > 1:
        lines += [f"- sum over the call's kernels: mean {sum(t[2] for t in timed):.2f} us, "
                  f"median {sum(t[3] for t in timed):.2f} us"]
    lines += [""]
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def _counter(d: str, kernel: str, counter: str):
    """Per-call value of a counter: for each kernel name matching the pattern,
    the median over its dispatches, summed over the matching kernels (a call
    that launches several kernels launches each once)."""
    pat = re.compile(kernel)
    by = {}
    for r in _rows(d, "counter_collection.csv"):
        if r["Counter_Name"] == counter and pat.search(r["Kernel_Name"]):
            key = (r["_file"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per = by.setdefault(r["Kernel_Name"], {})
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not by:
        sys.exit(f"no {counter} rows for {kernel} under {d}")
    return [sum(statistics.median(v.values()) for v in by.values())], \
        {name: statistics.median(v.values()) for name, v in by.items()}


def traffic(a):
    copy_bytes = 512 << 20
    fetch, fetch_by = _counter(a.fetch, a.kernel, "FETCH_SIZE")
    write, write_by = _counter(a.write, a.kernel, "WRITE_SIZE")
    cf, _ = _counter(a.calib_fetch, a.calib_kernel, "FETCH_SIZE")
    cw, _ = _counter(a.calib_write, a.calib_kernel, "WRITE_SIZE")
    f_fetch = copy_bytes / (statistics.median(cf) * 1024.0)
    f_write = copy_bytes / (statistics.median(cw) * 1024.0)
    rd = statistics.median(fetch) * 1024.0 * f_fetch
    wr = statistics.median(write) * 1024.0 * f_write
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash
    rec = {"kernel": a.name, "workload": a.workload, "hbm_bytes_per_launch": round(rd + wr),
           "read_bytes_per_launch": round(rd), "write_bytes_per_launch": round(wr),
           "fetch_size_kib_median": statistics.median(fetch),
           "write_size_kib_median": statistics.median(write),
           "per_kernel_fetch_kib": fetch_by, "per_kernel_write_kib": write_by,
           "copy_calibration": {"bytes": copy_bytes, "fetch_size_kib": statistics.median(cf),
                                "write_size_kib": statistics.median(cw),
                                "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
           "kernel_source_hash": kernel_source_hash(a.name)}
    with open(a.out_json, "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic of {a.name} on {a.workload} (rocprofv3 counters)", "",
             "Commands (from the repository root; one counter per run):", ""]
    lines += [f"    {c}" for c in a.command]
    lines += ["", f"- per call (median per kernel, summed over the call's kernels): FETCH_SIZE "
              f"{statistics.median(fetch):.0f} KiB, WRITE_SIZE {statistics.median(write):.0f} KiB"]
    lines += [f"  - `{n[:90]}`: FETCH_SIZE {fetch_by[n]:.0f} KiB, WRITE_SIZE {write_by.get(n, 0):.0f} KiB"
              for n in fetch_by]
    lines += [
              f"- copy calibration (elementwise copy of {copy_bytes} B): FETCH_SIZE "
              f"{statistics.median(cf):.0f} KiB, WRITE_SIZE {statistics.median(cw):.0f} KiB -> "
              f"factors {f_fetch:.4f} (fetch), {f_write:.4f} (write)",
              f"- scaled HBM bytes per launch: read {rd / 1e6:.2f} MB + write {wr / 1e6:.2f} MB = "
              f"{(rd + wr) / 1e6:.2f} MB", f"- kernel source hash: {rec['kernel_source_hash']}", ""]
    with open(a.out_txt, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def counters(a):
    """Median per-dispatch value of every collected counter for the kernels
    matching the pattern, with the MFMA utilisation and issued bf16 MFMA
    flops derived from them (GRBM_GUI_ACTIVE is summed over the XCDs in the
    CSV, so one XCD's active cycles are its value divided by the XCD count;
    SQ_VALU_MFMA_BUSY_CYCLES is summed over every SIMD)."""
    pat = re.compile(a.kernel)
    by = {}   # counter -> kernel -> dispatch -> value
    names = set()
    for d in a.dir:
        for r in _rows(d, "counter_collection.csv"):
            if not pat.search(r["Kernel_Name"]):
                continue
            names.add(r["Kernel_Name"])
            key = (r["_file"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per = by.setdefault(r["Counter_Name"], {}).setdefault(r["Kernel_Name"], {})
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not by:
        sys.exit(f"no counter rows for {a.kernel}")
    # per call: the median over a kernel's dispatches, summed over the
    # matching kernels (one call launches each of them once)
    med = {c: sum(statistics.median(v.values()) for v in ks.values()) for c, ks in by.items()}
    n = {c: max(len(v) for v in ks.values()) for c, ks in by.items()}
    lines = [f"# rocprofv3 counters: {a.title}", "", "Commands (from the repository root; one counter group per run):", ""]
    lines += [f"    {c}" for c in a.command]
    lines += ["", f"Kernel(s): {', '.join('`' + k[:100] + '`' for k in sorted(names))}", "",
              "| counter | per call (median per kernel, summed) | dispatches per kernel |", "|---|---|---|"]
    lines += [f"| {c} | {med[c]:.6g} | {n[c]} |" for c in sorted(med)]
    derived = {}
    if "GRBM_GUI_ACTIVE" in med:
        xcd_cycles = med["GRBM_GUI_ACTIVE"] / a.xcds
        derived["active cycles per XCD"] = f"{xcd_cycles:.0f} ({xcd_cycles / a.clock_ghz / 1e3:.1f} us at {a.clock_ghz} GHz)"
        if "TA_BUSY_avr" in med:
            derived["texture-address unit busy (TA_BUSY_avr / active cycles)"] = \
                f"{100 * med['TA_BUSY_avr'] / xcd_cycles:.1f} %"
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            u = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * a.simds)
            derived["MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x SIMDs))"] = f"{100 * u:.1f} %"
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
        derived["bf16 MFMA flops issued (MOPS x 512)"] = f"{med['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4g}"
    if "SQ_INSTS_VALU_MFMA_MOPS_F32" in med:
        derived["fp32 MFMA flops issued (MOPS x 512)"] = f"{med['SQ_INSTS_VALU_MFMA_MOPS_F32'] * 512:.4g}"
    if "SQ_WAVE_CYCLES" in med:
        wc = med["SQ_WAVE_CYCLES"]
        for c in ("SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
                  "SQ_ACTIVE_INST_VALU", "SQ_WAIT_ANY"):
            if c in med:
                derived[f"{c} / SQ_WAVE_CYCLES"] = f"{100 * med[c] / wc:.1f} %"
    if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med and med["SQ_LDS_IDX_ACTIVE"]:
        derived["LDS bank conflict / LDS active"] = f"{100 * med['SQ_LDS_BANK_CONFLICT'] / med['SQ_LDS_IDX_ACTIVE']:.1f} %"
    if derived:
        lines += ["", "Derived:", ""] + [f"- {k}: {v}" for k, v in derived.items()]
    sys.path.insert(0, ROOT)
    if a.source_key:
        from bench import kernel_source_hash
        lines += ["", f"Kernel source hash ({a.source_key}): {kernel_source_hash(a.source_key)}"]
    lines += [""]
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--steps", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    c = sub.add_parser("traffic")
    for k in ("fetch", "write", "calib_fetch", "calib_write", "kernel", "name", "workload",
              "out_json", "out_txt"):
        c.add_argument("--" + k.replace("_", "-"), required=True)
    c.add_argument("--calib-kernel", default="Mul")
    c.add_argument("--command", action="append", required=True)
    k = sub.add_parser("counters")
    k.add_argument("--dir", action="append", required=True)
    k.add_argument("--kernel", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--command", action="append", required=True)
    k.add_argument("--source-key", default=None, help="bench.KERNEL_SOURCES key whose hash to record")
    k.add_argument("--xcds", type=int, default=8)
    k.add_argument("--simds", type=int, default=1024)
    k.add_argument("--clock-ghz", type=float, default=2.4)
    a = ap.parse_args()
    {"trace": trace, "traffic": traffic, "counters": counters}[a.mode](a)


if __name__ == "__main__":
    main()
