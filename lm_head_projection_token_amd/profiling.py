"""Summaries of rocprofv3 output for the fused lm_head loss.

Usage (from the repository root, after the rocprofv3 runs):

  python -m lm_head_projection_token_amd.profiling kernels \\
      --stats DIR/NAME_kernel_stats.csv --workload W --command "..." --out profiles/X.md
  python -m lm_head_projection_token_amd.profiling traffic \\
      --fetch DIR_F --write DIR_W --copy-fetch DIR_CF --copy-write DIR_CW \\
      --copy-bytes N --workload W --command "..." --out profiles/Y

The traffic summary reads FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of
every library kernel, scales each counter by the factor that makes it read
right on a plain copy kernel of known size, and stores the per-launch HBM
bytes with a hash of the kernel sources. bench.py reports these bytes as
the dominant kernel's traffic only while the sources still hash the same.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# Kernel-name fragments -> the short names bench.py uses.
KINDS = [
    ("EpiLogits", "logits"), ("EpiDx", "dx"), ("EpiDw", "dw"),
    ("gemm_f32_kernel", "gemm_fp32"), ("row_kernel", "row"),
    ("dx_reduce_kernel", "dx_reduce"), ("colsum_kernel", "db"),
    ("finalize_kernel", "final"), ("prep_kernel", "prep"), ("fill_kernel", "fill"),
]


def kernel_kind(name: str) -> str | None:
    for frag, kind in KINDS:
        if frag in name:
            return kind
    return None


def source_hash() -> str:
    """sha256 over every kernel source file (any edit changes it)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def per_dispatch(d: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (summed over
    instances of the same dispatch)."""
    acc = defaultdict(float)
    names = {}
    for r in _counter_rows(d):
        if not r["Counter_Name"].startswith(counter):
            continue
        key = int(r["Dispatch_Id"])
        acc[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = defaultdict(list)
    for key in sorted(acc):
        out[names[key]].append(acc[key])
    return out


def copy_factor(d: str, counter: str, copy_bytes: int) -> float:
    """Expected bytes / counted bytes for the largest kernel in a copy run."""
    vals = per_dispatch(d, counter)
    best = max(vals.items(), key=lambda kv: statistics.median(kv[1]))
    counted = statistics.median(best[1]) * 1024.0
    return copy_bytes / counted


def kernels_summary(stats_csv: str, workload: str, command: str, out: str,
                    note: str = "") -> None:
    with open(stats_csv) as fh:
        rows = list(csv.DictReader(fh))
    lines = [f"# Kernel trace: {workload}", "",
             f"Command (from the repository root): `{command}`", "",
             "| kernel | calls | average (ms) | total (ms) | share |",
             "|---|---|---|---|---|"]
    for r in rows:
        kind = kernel_kind(r["Name"])
        if kind is None:
            continue
        lines.append(f"| {kind} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}% |")
    if note:
        lines += ["", note]
    lines += ["", f"Kernel sources sha256: `{source_hash()}`", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))


def traffic_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes,
                    workload, command, out_base) -> None:
    ff = copy_factor(copy_fetch_dir, "FETCH_SIZE", copy_bytes)
    wf = copy_factor(copy_write_dir, "WRITE_SIZE", copy_bytes)
    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    kinds = {}
    for name, vals in fetch.items():
        kind = kernel_kind(name)
        if kind is None or name not in write:
            continue
        fb = statistics.median(vals) * 1024.0 * ff
        wb = statistics.median(write[name]) * 1024.0 * wf
        kinds[kind] = {"fetch_bytes": fb, "write_bytes": wb, "dispatches": len(vals)}
    rec = {"workload": workload, "command": command, "copy_bytes": copy_bytes,
           "copy_fetch_factor": ff, "copy_write_factor": wf,
           "src_sha256": source_hash(), "kernels": kinds}
    with open(out_base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = [f"# HBM traffic per launch: {workload}", "",
             f"Commands (from the repository root): {command}", "",
             f"Copy calibration: a {copy_bytes / 2**30:.2f} GiB device copy reads "
             f"FETCH_SIZE x {ff:.4f} and WRITE_SIZE x {wf:.4f} of its true bytes; "
             "both factors are applied below.", "",
             "| kernel | fetched (GB) | written (GB) | dispatches |", "|---|---|---|---|"]
    for k, v in sorted(kinds.items()):
        lines.append(f"| {k} | {v['fetch_bytes'] / 1e9:.3f} | {v['write_bytes'] / 1e9:.3f} | "
                     f"{v['dispatches']} |")
    lines += ["", f"Kernel sources sha256: `{rec['src_sha256']}`", ""]
    with open(out_base + ".md", "w") as fh:
        fh.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("--stats", required=True)
    k.add_argument("--workload", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload",
              "--command", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    args = ap.parse_args()
    if args.cmd == "kernels":
        kernels_summary(args.stats, args.workload, args.command, args.out, args.note)
    else:
        traffic_summary(args.fetch, args.write, args.copy_fetch, args.copy_write,
                        args.copy_bytes, args.workload, args.command, args.out)


if __name__ == "__main__":
    main()
