"""Benchmark: fused lm_head loss, fwd+bwd tokens/s on one MI355X.

A step is one ``fll_fwd_bwd`` call over the whole batch: every token chunk's
logits GEMM, fused row kernel, dX GEMM (+ split reduction) and, for trainable
heads, the dW / db kernels, then the loss reduction. Inputs are synthetic,
seeded, and resident in HBM before timing starts.

Default workload: GRPO selective log-prob with a frozen head, B=8, T=1024
(BT = 8192 tokens), H = 4096, V = 128256, bf16 -- the head shape and batch
the frozen lm_head GRPO page times (Details). ``--config 5`` selects the
trainable KL distillation workload at the same H and V, ``--config jsd`` the
Jensen-Shannon head against a teacher with its own H = 4096 projection,
``--config ppo`` the PPO clipped surrogate on the default workload's shape
(its old log-probs are -log V minus the drawn log-ratios: the work per row
does not depend on which clip branch a row takes).

Prints one JSON line. ``value`` and ``ms_per_step`` come from the timed
steps alone; ``kernels`` and ``roofline`` (the dominant kernel) from as many
steps again with HIP events around every kernel on the library's stream, so
the events' own cost stays out of the step time; ``cpu_baseline``
times the CPU float64 oracle on a bounded row sample and extrapolates
linearly in rows (every step of the method is row-local except the final
sum).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "fwd+bwd tokens/sec at H=4096,V=128256 bf16; % of bf16 MFMA peak"
COPY_BYTES = 1 << 30


def measured_traffic(case, kind, logits_bf16=False):
    """HBM bytes per launch of `kind` from the committed counter summary of
    this workload (and chunk-logits type), or None if there is none or the
    kernels changed since."""
    from lm_head_projection_token_amd import profiling

    tag = case.name + ("-bf16-logits" if logits_bf16 else "")
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("src_sha256") != profiling.source_hash():
        return None
    k = rec.get("kernels", {}).get(kind)
    if not k:
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def measured_clock(case, kind, logits_bf16=False):
    """Shader clock (GHz) and MFMA busy fraction of `kind` from the committed
    counter summary of this workload (GRBM_COUNT over the kernel's duration),
    or None if there is none or the kernels changed since."""
    from lm_head_projection_token_amd import profiling

    tag = case.name + ("-bf16-logits" if logits_bf16 else "")
    path = os.path.join(ROOT, "profiles", f"mfma_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("src_sha256") != profiling.source_hash():
        return None
    k = rec.get("kernels", {}).get(kind)
    if not k or not k.get("clock_GHz"):
        return None
    return k["clock_GHz"], k.get("mfma_busy")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def gemm_flops(case):
    """Algorithmic flops of one step: logits and dX GEMMs, plus dW if formed,
    plus the teacher's logits GEMM for the JSD head."""
    f = 4.0 * case.BT * case.H * case.V
    if case.compute_dW:
        f += 2.0 * case.BT * case.H * case.V
    if case.head == "jsd":
        f += 2.0 * case.BT * case.H_teacher * case.V
    return f


def kernel_flops(kind, case):
    per = 2.0 * case.BT * case.H * case.V
    return {"logits": per, "dx": per, "dw": per if case.compute_dW else 0.0,
            "teacher": 2.0 * case.BT * case.H_teacher * case.V}.get(kind, 0.0)


def gemm_bytes_per_launch(kind, case, n_chunks, logits_bf16=False):
    """Algorithmic HBM bytes of one launch of a GEMM (a chunk of BT/n_chunks
    rows on average): each operand read once and each output written once.
    logits / teacher: X chunk, W (and b) read, the chunk's logits (4 or 2
    bytes each) and its per-(row, 128-column) statistics written; dX: the
    bf16 dZ chunk and W read, dX written; dW: the bf16 dZ chunk and the
    chunk's X read, fp32 dW written, and read back on every chunk after the
    first (averaged over the chunks)."""
    es = 2 if case.dtype == "bf16" else 4
    C = case.BT / max(n_chunks, 1)
    V = case.V
    nstat = -(-V // 128)
    s = 2 if logits_bf16 else 4
    if kind in ("logits", "teacher"):
        Hk = case.H if kind == "logits" else case.H_teacher
        bias = case.has_bias if kind == "logits" else case.teacher_has_bias
        return C * Hk * es + V * Hk * es + (V * es if bias else 0) + C * V * s + C * nstat * 8
    if kind == "dx":
        return C * V * es + V * case.H * es + C * case.H * es
    if kind == "dw":
        old = (n_chunks - 1) / max(n_chunks, 1)
        return C * V * es + C * case.H * es + V * case.H * 4 * (1 + old)
    return 0.0


def row_bytes_per_valid_row(case, logits_bf16=False):
    """Algorithmic HBM bytes of the row kernel per valid row: one read of the
    logits (and of the fp32 target or the teacher's logits) and one write of
    the bf16 dZ; logits are 4 bytes each, or 2 when kept in bf16."""
    s = 2 if logits_bf16 else 4
    extra = {"kl": 4, "jsd": s}.get(case.head, 0)
    return (s + extra + 2) * case.V


def sample_clock(step, sync, ms_per_step, samples=6):
    """Shader clock (GHz) while steps run back to back: `amd-smi metric
    --clock` is read a few times from a helper thread, each reading averaged
    over the GFX clock of every XCD. Steps are queued ~100 ms at a time so
    that the GPU does not idle between them while a reading is taken. Returns (mean, min, max) of the
    readings and their count, or None if amd-smi is missing or prints no GFX clock. amd-smi
    refreshes the figure slowly (readings of one run can repeat exactly), and
    it mixes GEMM and row-kernel phases;
    the per-kernel clocks come from the counters (GRBM_COUNT)."""
    import re
    import shutil
    import subprocess
    import threading

    exe = shutil.which("amd-smi")
    if not exe:
        return None
    readings = []
    done = threading.Event()

    def sampler():
        try:
            time.sleep(0.3)
            for _ in range(samples):
                out = subprocess.run([exe, "metric", "-g", "0", "--clock"], capture_output=True,
                                     text=True, timeout=20).stdout
                mhz = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", out)]
                if mhz:
                    readings.append(sum(mhz) / len(mhz))
        except Exception:  # pragma: no cover - a reading is optional
            pass
        finally:
            done.set()

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t_end = time.perf_counter() + 60.0
    batch = max(10, int(100.0 / max(ms_per_step, 1e-3)))
    while not done.is_set() and time.perf_counter() < t_end:
        for _ in range(batch):
            step()
        sync()
    th.join(timeout=30)
    if not readings:
        return None
    return (sum(readings) / len(readings) / 1e3, min(readings) / 1e3, max(readings) / 1e3,
            len(readings))


def clock_record(clk, case, ms, achieved):
    """The clock object of the JSON line from sample_clock's readings. A
    reading whose peak at that clock is below what the dominant kernel was
    measured to reach cannot be the clock it ran at (amd-smi can report a
    stale or idle value while short kernels run), and readings that repeat
    to the kHz are amd-smi's slowly refreshed figure, not the clock of the
    steps: in both cases no fraction is derived from them and the record
    says why (the per-kernel clock of ``roofline`` comes from counters)."""
    ghz = clk[0]
    peak_at_clock = (PEAK_BF16_TFLOPS if case.dtype == "bf16" else PEAK_FP32_TFLOPS) * ghz / 2.4
    rec = {"source": "amd-smi metric --clock (GFX clock averaged over the XCDs) while "
                     "steps ran back to back after the timed region",
           "GHz": ghz, "GHz_min": clk[1], "GHz_max": clk[2], "readings": clk[3]}
    if achieved > peak_at_clock:
        rec.update(GHz=None, discarded_GHz=ghz,
                   note="readings below the clock the measured throughput needs; discarded")
        return rec
    if clk[3] > 1 and clk[1] == clk[2]:
        rec["note"] = ("every reading identical: a stale amd-smi figure, so no fraction "
                       "at this clock is given")
        return rec
    rec.update(peak_at_clock=peak_at_clock,
               end_to_end_frac_at_clock=gemm_flops(case) / (ms / 1e3) / 1e12 / peak_at_clock,
               roofline_frac_at_clock=achieved / peak_at_clock)
    return rec


def cpu_baseline(inp, case, rows_small=256, rows_big=3072, old=None):
    """Time the oracle on two row samples and extrapolate to the full batch."""
    import numpy as np

    from oracle import fll_oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count()

    Wd = inp["W"]
    bd = inp["b"]
    Wt = None if inp["W_teacher"] is None else inp["W_teacher"].double().numpy()
    bt = None if inp["b_teacher"] is None else inp["b_teacher"].double().numpy()

    def run(R):
        rows = np.arange(R)
        X = inp["X"][:R].double().numpy()
        t0 = time.perf_counter()
        fll_oracle.sampled_rows(
            X, Wd.double().numpy(), None if bd is None else bd.double().numpy(),
            head=case.head, n_valid=case.BT,
            labels_rows=None if inp["labels"] is None else inp["labels"][rows].numpy(),
            target_rows=None if inp["target"] is None else inp["target"][:R].double().numpy(),
            weights_rows=None if inp["weights"] is None else inp["weights"][:R].double().numpy(),
            reduction=case.reduction, ignore_index=case.ignore_index,
            temperature=case.temperature, eps=case.eps,
            Xt_rows=None if inp["X_teacher"] is None else inp["X_teacher"][:R].double().numpy(),
            W_teacher=Wt, b_teacher=bt,
            old_logprobs_rows=None if old is None else old[:R].double().numpy(),
            clip_low=case.clip_low, clip_high=case.clip_high)
        return time.perf_counter() - t0

    t1 = run(rows_small)
    t2 = run(rows_big)
    per_row = max((t2 - t1) / (rows_big - rows_small), 1e-12)
    fixed = max(t1 - per_row * rows_small, 0.0)
    est = fixed + per_row * case.BT
    return {
        "value": case.BT / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"numpy float64 oracle (sampled_rows: logits, log-softmax, loss terms, "
                   f"dlogits, dX{', teacher logits' if case.head == 'jsd' else ''}) timed on "
                   f"the first {rows_small} and {rows_big} token rows "
                   f"({t1:.2f} s, {t2:.2f} s), extrapolated linearly to BT={case.BT}"
                   + ("; the dW GEMM is not in the sample" if case.compute_dW else "")),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="3", choices=["2", "3", "4", "5", "jsd", "ppo"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--logits-bf16", action="store_true",
                    help="keep each chunk's logits in bf16 instead of fp32")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the amd-smi shader-clock reading after the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch

        n = COPY_BYTES // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # reads and writes COPY_BYTES
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the fused lm_head loss is a single-GPU "
              "operator here; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import lm_head_projection_token_amd as fll
    import workloads

    named = {"jsd": workloads.JSD_WORKLOAD, "ppo": workloads.PPO_WORKLOAD}
    case = named[args.config] if args.config in named else workloads.WORKLOADS[int(args.config)]
    inp = workloads.make_inputs(case)
    old = None
    if case.head in workloads.RATIO_HEADS:
        # synthetic old log-probs: the time per row does not depend on them
        old = -math.log(case.V) - inp["logratio"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(t):
        return None if t is None else t.to(dev).contiguous()

    X, W, b = d(inp["X"]), d(inp["W"]), d(inp["b"])
    labels, target, weights = d(inp["labels"]), d(inp["target"]), d(inp["weights"])
    Xt, Wt, bt = d(inp["X_teacher"]), d(inp["W_teacher"]), d(inp["b_teacher"])
    old_d = d(old)
    prob = fll.make_problem(case.BT, case.H, case.V, dtype=case.dtype, head=case.head,
                            has_bias=case.has_bias, compute_dW=case.compute_dW,
                            compute_db=case.compute_db, reduction=case.reduction,
                            ignore_index=case.ignore_index, temperature=case.temperature,
                            eps=case.eps, H_teacher=case.H_teacher,
                            teacher_has_bias=case.teacher_has_bias,
                            logits_bf16=args.logits_bf16,
                            clip_low=case.clip_low if old is not None else None,
                            clip_high=case.clip_high if old is not None else None)
    plan = fll.fll_plan(prob, 0, args.chunk_rows)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    dX = torch.empty_like(X)
    dW = torch.empty(case.V, case.H, dtype=torch.float32, device=dev) if case.compute_dW else None
    db = torch.empty(case.V, dtype=torch.float32, device=dev) if case.compute_db else None
    loss = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        fll.fll_fwd_bwd(plan, X=X, W=W, b=b, labels=labels, target=target, weights=weights,
                        dX=dX, dW=dW, db=db, loss=loss, workspace=ws, stream=stream,
                        X_teacher=Xt, W_teacher=Wt, b_teacher=bt, old_logprobs=old_d)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)

    # The steps themselves, with no per-kernel events (each event adds a few
    # microseconds at a kernel boundary: ~10 % of a V=32000 step).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    # The same number of steps again with the library's HIP events around
    # every kernel, on its launch stream: the per-kernel times and roofline.
    fll.fll_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = fll.fll_profile_read(reset=True)
    fll.fll_profile_enable(False)
    if not torch.isfinite(loss):
        raise RuntimeError("non-finite loss")

    tokens_per_s = case.BT / (ms / 1e3)
    peak = PEAK_BF16_TFLOPS if case.dtype == "bf16" else PEAK_FP32_TFLOPS
    e2e_frac = gemm_flops(case) / (ms / 1e3) / 1e12 / peak

    kernels = {}
    for kind, (n, tot) in prof.items():
        if n:
            kernels[kind] = {"launches": n, "avg_ms": tot / n, "ms_per_step": tot / args.steps}
    gemms = [k for k in ("logits", "dx", "dw", "teacher") if k in kernels]
    dom = max(gemms, key=lambda k: kernels[k]["ms_per_step"])
    per_launch = kernel_flops(dom, case) / plan.n_chunks
    achieved = per_launch / (kernels[dom]["avg_ms"] / 1e3) / 1e12
    # the teacher's logits GEMM is the logits kernel: the counter summaries
    # (by kernel) hold it under that name, averaged with the student's
    prof_kind = "logits" if dom == "teacher" else dom
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": measured_traffic(case, prof_kind, args.logits_bf16),
                "flops_per_launch": per_launch,
                "algorithmic_bytes_per_launch": gemm_bytes_per_launch(
                    dom, case, plan.n_chunks, args.logits_bf16)}
    clk = measured_clock(case, prof_kind, args.logits_bf16)
    if clk:
        # the clock this kernel ran at, from the committed counter summary
        # (GRBM_COUNT over the kernel's duration) of the same kernel sources
        roofline.update(counter_clock_GHz=clk[0], counter_mfma_busy=clk[1],
                        frac_at_counter_clock=achieved / (peak * clk[0] / 2.4))
    row = kernels.get("row")
    if row:
        bytes_per_row = row_bytes_per_valid_row(case, args.logits_bf16)
        n_valid = case.BT if inp["labels"] is None else int(
            (inp["labels"] != case.ignore_index).sum())
        row_bytes = bytes_per_row * n_valid / plan.n_chunks
        kernels["row"]["achieved_GBps"] = row_bytes / (row["avg_ms"] / 1e3) / 1e9

    out = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": case.name, "BT": case.BT, "H": case.H, "V": case.V,
                   "head": case.head, **({"H_teacher": case.H_teacher} if case.head == "jsd" else {}), "compute_dW": case.compute_dW,
                   "compute_db": case.compute_db, "chunk_rows": plan.chunk_rows,
                   "n_chunks": plan.n_chunks,
                   "chunk_logits": "bf16" if args.logits_bf16 else "fp32",
                   "parallelism": "single GPU"},
        "end_to_end_frac_of_bf16_peak": e2e_frac,
        "wall_s": wall,
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_clock:
        # The chip's power limit sets the shader clock under this load; the
        # dense peak above assumes 2.4 GHz. Reported beside it, not instead.
        print("[bench] reading the shader clock while steps run", file=sys.stderr, flush=True)
        clk = sample_clock(step, torch.cuda.synchronize, ms)
        if clk:
            out["clock"] = clock_record(clk, case, ms, achieved)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, case, old=old)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
