"""Summaries of rocprofv3 output for the fused lm_head loss.

Usage (from the repository root, after the rocprofv3 runs):

  python -m lm_head_projection_token_amd.profiling kernels \\
      --stats DIR/NAME_kernel_stats.csv --workload W --command "..." --out profiles/X.md
  python -m lm_head_projection_token_amd.profiling traffic \\
      --fetch DIR_F --write DIR_W --copy-fetch DIR_CF --copy-write DIR_CW \\
      --copy-bytes N --workload W --command "..." --out profiles/Y
  python -m lm_head_projection_token_amd.profiling mfma \\
      --dir DIR_M --workload W --command "..." --out profiles/Z

The MFMA summary reads, per dispatch, SQ_VALU_MFMA_BUSY_CYCLES,
SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE and GRBM_COUNT (one --pmc run
with --kernel-trace, which gives each dispatch's duration) and reports the
shader clock the kernel ran at, the MFMA pipes' busy fraction and the bf16
MFMA flops counted by the hardware.

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
    ("transpose_bf16_kernel", "transpose"),
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


N_XCD = 8
N_CU = 256
N_SIMD = N_CU * 4
PEAK_CLOCK_GHZ = 2.4
FLOP_PER_CLK_SIMD_BF16 = 1024  # dense bf16: 256 CU x 4 SIMD x 1024 x 2.4 GHz = 2516.6 TFLOP/s


def _trace_durations(d: str):
    """{dispatch id: (kernel name, duration in ns)} from a kernel trace."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {d}")
    out = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out[int(r["Dispatch_Id"])] = (
                    r["Kernel_Name"], float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return out


def mfma_summary(d, workload, command, out_base) -> None:
    """Per kernel kind (median over dispatches): duration, shader clock
    (GRBM_COUNT per XCD over the duration), busy clock (GRBM_GUI_ACTIVE per
    XCD), MFMA busy fraction of every SIMD's active cycles, and the bf16 MFMA
    flops the hardware counted, as TFLOP/s and as fractions of the dense peak
    at 2.4 GHz and at the measured clock."""
    names = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE",
             "GRBM_COUNT")
    vals = defaultdict(lambda: defaultdict(float))
    for r in _counter_rows(d):
        n = r["Counter_Name"]
        if n in names:
            vals[int(r["Dispatch_Id"])][n] += float(r["Counter_Value"])
    durs = _trace_durations(d)
    per_kind = defaultdict(list)
    for did, c in vals.items():
        if did not in durs or any(n not in c for n in names):
            continue
        kname, ns = durs[did]
        kind = kernel_kind(kname)
        if kind is None or ns <= 0:
            continue
        clk = c["GRBM_COUNT"] / N_XCD / ns          # cycles per ns = GHz
        active = c["GRBM_GUI_ACTIVE"] / N_XCD
        util = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * N_SIMD) if active else 0.0
        tflops = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / ns / 1e3
        peak_nominal = N_SIMD * FLOP_PER_CLK_SIMD_BF16 * PEAK_CLOCK_GHZ / 1e3
        peak_clock = N_SIMD * FLOP_PER_CLK_SIMD_BF16 * clk / 1e3
        per_kind[kind].append({"duration_ms": ns / 1e6, "clock_GHz": clk,
                               "active_GHz": active / ns, "mfma_busy": util,
                               "mfma_TFLOPs": tflops, "frac_peak": tflops / peak_nominal,
                               "frac_peak_at_clock": tflops / peak_clock if clk else 0.0})
    kinds = {}
    for kind, rows in per_kind.items():
        kinds[kind] = {k: statistics.median(r[k] for r in rows) for k in rows[0]}
        kinds[kind]["dispatches"] = len(rows)
    rec = {"workload": workload, "command": command, "src_sha256": source_hash(),
           "kernels": kinds}
    with open(out_base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = [f"# MFMA utilisation and shader clock: {workload}", "",
             f"Command (from the repository root): `{command}`", "",
             "Per dispatch: clock = GRBM_COUNT / 8 XCDs / duration; MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); bf16 "
             "TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration (hardware-counted "
             "MFMA flops, tail and padding included). Medians over dispatches; "
             "durations are from the counter run, where dispatches are serialised.", "",
             "| kernel | dispatches | duration (ms) | clock (GHz) | MFMA busy | "
             "bf16 TFLOP/s | of peak at 2.4 GHz | of peak at the clock |",
             "|---|---|---|---|---|---|---|---|"]
    for k, v in sorted(kinds.items(), key=lambda kv: -kv[1]["duration_ms"]):
        lines.append(f"| {k} | {v['dispatches']} | {v['duration_ms']:.4f} | "
                     f"{v['clock_GHz']:.3f} | {100 * v['mfma_busy']:.1f}% | "
                     f"{v['mfma_TFLOPs']:.1f} | {100 * v['frac_peak']:.1f}% | "
                     f"{100 * v['frac_peak_at_clock']:.1f}% |")
    lines += ["", f"Kernel sources sha256: `{rec['src_sha256']}`", ""]
    with open(out_base + ".md", "w") as fh:
        fh.write("\n".join(lines))


def lds_summary(d, workload, command, out_base) -> None:
    """Per kernel kind (median over dispatches): LDS instructions issued per
    CU, the cycles the LDS spent on indexed (ds_read / ds_write) work and the
    cycles it stalled on bank conflicts, both per CU, and conflicts as a
    fraction of the indexed cycles."""
    names = ("SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT")
    vals = defaultdict(lambda: defaultdict(float))
    kname = {}
    for r in _counter_rows(d):
        n = r["Counter_Name"]
        if n in names:
            vals[int(r["Dispatch_Id"])][n] += float(r["Counter_Value"])
            kname[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    per_kind = defaultdict(list)
    for did, c in vals.items():
        kind = kernel_kind(kname[did])
        if kind is None or any(n not in c for n in names):
            continue
        idx = c["SQ_LDS_IDX_ACTIVE"]
        per_kind[kind].append({"lds_insts_per_cu": c["SQ_INSTS_LDS"] / N_CU,
                               "idx_active_per_cu": idx / N_CU,
                               "bank_conflict_per_cu": c["SQ_LDS_BANK_CONFLICT"] / N_CU,
                               "conflict_frac": c["SQ_LDS_BANK_CONFLICT"] / idx if idx else 0.0})
    kinds = {}
    for kind, rows in per_kind.items():
        kinds[kind] = {k: statistics.median(r[k] for r in rows) for k in rows[0]}
        kinds[kind]["dispatches"] = len(rows)
    rec = {"workload": workload, "command": command, "src_sha256": source_hash(),
           "kernels": kinds}
    with open(out_base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = [f"# LDS bank conflicts: {workload}", "",
             f"Command (from the repository root): `{command}`", "",
             "Per dispatch, divided by 256 CUs: SQ_INSTS_LDS (LDS instructions issued), "
             "SQ_LDS_IDX_ACTIVE (cycles of indexed LDS work), SQ_LDS_BANK_CONFLICT "
             "(cycles stalled on bank conflicts); conflict share = bank-conflict cycles / "
             "indexed cycles. Medians over dispatches.", "",
             "| kernel | dispatches | LDS insts per CU | indexed cycles per CU | "
             "conflict cycles per CU | conflict share |",
             "|---|---|---|---|---|---|"]
    for k, v in sorted(kinds.items(), key=lambda kv: -kv[1]["idx_active_per_cu"]):
        lines.append(f"| {k} | {v['dispatches']} | {v['lds_insts_per_cu']:.0f} | "
                     f"{v['idx_active_per_cu']:.0f} | {v['bank_conflict_per_cu']:.0f} | "
                     f"{100 * v['conflict_frac']:.2f}% |")
    lines += ["", f"Kernel sources sha256: `{rec['src_sha256']}`", ""]
    with open(out_base + ".md", "w") as fh:
        fh.write("\n".join(lines))


def ta_summary(d, workload, command, out_base) -> None:
    """Per kernel kind (median over dispatches): the fraction of active
    cycles the texture-address (TA) unit of a CU is busy, TA_BUSY_avr (TA
    busy cycles averaged over the TA instances) over GRBM_GUI_ACTIVE / 8 XCDs,
    and the buffer-instruction share of those cycles,
    TA_BUFFER_TOTAL_CYCLES_sum / (TA_BUSY_avr x 256 instances)."""
    names = ("TA_BUSY_avr", "TA_BUFFER_TOTAL_CYCLES_sum", "GRBM_GUI_ACTIVE")
    vals = defaultdict(lambda: defaultdict(float))
    kname = {}
    for r in _counter_rows(d):
        n = r["Counter_Name"]
        if n in names:
            vals[int(r["Dispatch_Id"])][n] += float(r["Counter_Value"])
            kname[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    per_kind = defaultdict(list)
    for did, c in vals.items():
        kind = kernel_kind(kname[did])
        if kind is None or any(n not in c for n in names):
            continue
        active = c["GRBM_GUI_ACTIVE"] / N_XCD
        busy = c["TA_BUSY_avr"]
        per_kind[kind].append({
            "ta_busy_frac": busy / active if active else 0.0,
            "buffer_share": c["TA_BUFFER_TOTAL_CYCLES_sum"] / (busy * N_CU) if busy else 0.0})
    kinds = {}
    for kind, rows in per_kind.items():
        kinds[kind] = {k: statistics.median(r[k] for r in rows) for k in rows[0]}
        kinds[kind]["dispatches"] = len(rows)
    rec = {"workload": workload, "command": command, "src_sha256": source_hash(),
           "kernels": kinds}
    with open(out_base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = [f"# Texture-address unit busy: {workload}", "",
             f"Command (from the repository root): `{command}`", "",
             "Per dispatch: TA busy = TA_BUSY_avr / (GRBM_GUI_ACTIVE / 8 XCDs), the share of "
             "active cycles a CU's TA unit (address processing of every vector memory "
             "instruction, LDS-DMA loads included) is busy; buffer share = "
             "TA_BUFFER_TOTAL_CYCLES_sum / (TA_BUSY_avr x 256). Medians over dispatches.", "",
             "| kernel | dispatches | TA busy | buffer share of TA cycles |",
             "|---|---|---|---|"]
    for k, v in sorted(kinds.items(), key=lambda kv: -kv[1]["ta_busy_frac"]):
        lines.append(f"| {k} | {v['dispatches']} | {100 * v['ta_busy_frac']:.1f}% | "
                     f"{100 * v['buffer_share']:.1f}% |")
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
    m = sub.add_parser("mfma")
    for a in ("--dir", "--workload", "--command", "--out"):
        m.add_argument(a, required=True)
    ls = sub.add_parser("lds")
    for a in ("--dir", "--workload", "--command", "--out"):
        ls.add_argument(a, required=True)
    ta = sub.add_parser("ta")
    for a in ("--dir", "--workload", "--command", "--out"):
        ta.add_argument(a, required=True)
    args = ap.parse_args()
    if args.cmd == "ta":
        ta_summary(args.dir, args.workload, args.command, args.out)
    elif args.cmd == "lds":
        lds_summary(args.dir, args.workload, args.command, args.out)
    elif args.cmd == "kernels":
        kernels_summary(args.stats, args.workload, args.command, args.out, args.note)
    elif args.cmd == "mfma":
        mfma_summary(args.dir, args.workload, args.command, args.out)
    else:
        traffic_summary(args.fetch, args.write, args.copy_fetch, args.copy_write,
                        args.copy_bytes, args.workload, args.command, args.out)


if __name__ == "__main__":
    main()
