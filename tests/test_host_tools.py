"""Host-side tools: bench.py's one-GPU guard, its flop / byte bookkeeping
and its CPU-oracle timing, the rocprofv3 summaries of the profiling module
on small synthetic CSV files, and the build entry point on a fresh checkout
(all without a GPU); and, marked gpu, bench.py's JSON line on a small
workload.
"""

import csv
import json
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from lm_head_projection_token_amd import profiling  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_bench_flops_follow_the_gradient_flags():
    frozen = workloads.WORKLOADS[3]
    trainable = workloads.WORKLOADS[5]
    per = 2.0 * frozen.BT * frozen.H * frozen.V
    # logits and dX only when frozen; dW adds a third product
    assert bench.gemm_flops(frozen) == 2 * per
    assert bench.gemm_flops(trainable) == 3 * 2.0 * trainable.BT * trainable.H * trainable.V
    assert bench.kernel_flops("dw", frozen) == 0.0
    assert bench.kernel_flops("logits", frozen) == per
    jsd = workloads.JSD_WORKLOAD
    assert bench.gemm_flops(jsd) == 2.0 * jsd.BT * jsd.V * (2 * jsd.H + jsd.H_teacher)


def test_bench_gemm_bytes_per_launch():
    # each operand read once, each output written once, per launch of a
    # 4096-row chunk (V = 128256, H = 4096, bf16)
    c3 = workloads.WORKLOADS[3]
    C, H, V = 4096, 4096, 128256
    assert bench.gemm_bytes_per_launch("logits", c3, 2) == \
        C * H * 2 + V * H * 2 + C * V * 4 + C * 1002 * 8
    assert bench.gemm_bytes_per_launch("logits", c3, 2, logits_bf16=True) == \
        C * H * 2 + V * H * 2 + C * V * 2 + C * 1002 * 8
    assert bench.gemm_bytes_per_launch("dx", c3, 2) == C * V * 2 + V * H * 2 + C * H * 2
    # dW of the two-chunk V = 151936 workload: fp32 dW written twice, read once
    c4 = workloads.WORKLOADS[4]
    V4 = 151936
    assert bench.gemm_bytes_per_launch("dw", c4, 2) == \
        C * V4 * 2 + C * H * 2 + V4 * H * 4 * 1.5


def test_bench_row_bytes_per_valid_row():
    V = workloads.WORKLOADS[3].V
    # selective: read fp32 logits, write bf16 dlogits; KL also reads the fp32 target
    assert bench.row_bytes_per_valid_row(workloads.WORKLOADS[3]) == 6 * V
    assert bench.row_bytes_per_valid_row(workloads.WORKLOADS[5]) == 10 * V
    assert bench.row_bytes_per_valid_row(workloads.WORKLOADS[3], logits_bf16=True) == 4 * V
    assert bench.row_bytes_per_valid_row(workloads.JSD_WORKLOAD) == 10 * V


def test_measured_traffic_needs_matching_sources(tmp_path, monkeypatch):
    case = workloads.WORKLOADS[3]
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"src_sha256": profiling.source_hash(),
           "kernels": {"logits": {"fetch_bytes": 3.0, "write_bytes": 4.0}}}
    (prof / f"traffic_{case.name}.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(case, "logits") == 7.0
    assert bench.measured_traffic(case, "dx") is None
    rec["src_sha256"] = "0" * 64  # counters taken on other kernel sources
    (prof / f"traffic_{case.name}.json").write_text(json.dumps(rec))
    assert bench.measured_traffic(case, "logits") is None


LOGITS = "fll::gemm_kernel<true, true, fll::EpiLogits<false>>(fll::GemmDesc, fll::EpiLogits<false>)"
ROW = "fll::row_kernel<1, false>(fll::RowArgs)"


def _write_counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    copy_bytes = 1 << 30
    d = {k: tmp_path / k for k in ("cf", "cw", "f", "w")}
    for p in d.values():
        p.mkdir()
    # the copy reads FETCH_SIZE = half its bytes and WRITE_SIZE = all of them (KiB)
    _write_counters(d["cf"] / "p_counter_collection.csv",
                    [{"Dispatch_Id": 1, "Kernel_Name": "copy", "Counter_Name": "FETCH_SIZE",
                      "Counter_Value": copy_bytes / 2 / 1024}])
    _write_counters(d["cw"] / "p_counter_collection.csv",
                    [{"Dispatch_Id": 1, "Kernel_Name": "copy", "Counter_Name": "WRITE_SIZE",
                      "Counter_Value": copy_bytes / 1024}])
    # two dispatches of the logits GEMM, each counter split over two instances
    rows_f, rows_w = [], []
    for did, kib in ((5, 1000.0), (9, 1200.0)):
        for half in (0.25, 0.75):
            rows_f.append({"Dispatch_Id": did, "Kernel_Name": LOGITS,
                           "Counter_Name": "FETCH_SIZE", "Counter_Value": kib * half})
            rows_w.append({"Dispatch_Id": did, "Kernel_Name": LOGITS,
                           "Counter_Name": "WRITE_SIZE", "Counter_Value": 10 * kib * half})
    _write_counters(d["f"] / "p_counter_collection.csv", rows_f)
    _write_counters(d["w"] / "p_counter_collection.csv", rows_w)
    out = tmp_path / "traffic_x"
    profiling.traffic_summary(str(d["f"]), str(d["w"]), str(d["cf"]), str(d["cw"]), copy_bytes,
                              "x", "cmd", str(out))
    rec = json.loads((tmp_path / "traffic_x.json").read_text())
    assert rec["copy_fetch_factor"] == pytest.approx(2.0)
    assert rec["copy_write_factor"] == pytest.approx(1.0)
    k = rec["kernels"]["logits"]
    # median over dispatches of the instance sums, in bytes, times the factors
    assert k["fetch_bytes"] == pytest.approx(1100.0 * 1024 * 2.0)
    assert k["write_bytes"] == pytest.approx(11000.0 * 1024 * 1.0)
    assert k["dispatches"] == 2
    assert "| logits |" in (tmp_path / "traffic_x.md").read_text()


def test_mfma_summary_clock_busy_and_flops(tmp_path):
    d = tmp_path / "m"
    d.mkdir()
    ns = 2.0e6  # a 2 ms dispatch
    ghz = 1.8
    busy = 0.7
    gui = ghz * ns  # active cycles per XCD
    rows = []
    for name, val in (("GRBM_COUNT", 8 * ghz * ns), ("GRBM_GUI_ACTIVE", 8 * gui),
                      ("SQ_VALU_MFMA_BUSY_CYCLES", busy * gui * 1024),
                      # flops counted by the hardware: MOPS x 512
                      ("SQ_INSTS_VALU_MFMA_MOPS_BF16", busy * gui * 1024 * 1024 / 512)):
        rows.append({"Dispatch_Id": 3, "Kernel_Name": LOGITS, "Counter_Name": name,
                     "Counter_Value": val})
    _write_counters(d / "m_counter_collection.csv", rows)
    with open(d / "m_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                           "End_Timestamp"])
        w.writeheader()
        w.writerow({"Dispatch_Id": 3, "Kernel_Name": LOGITS, "Start_Timestamp": 1000,
                    "End_Timestamp": 1000 + ns})
        w.writerow({"Dispatch_Id": 4, "Kernel_Name": ROW, "Start_Timestamp": 5000,
                    "End_Timestamp": 6000})
    profiling.mfma_summary(str(d), "x", "cmd", str(tmp_path / "mfma_x"))
    k = json.loads((tmp_path / "mfma_x.json").read_text())["kernels"]["logits"]
    assert k["clock_GHz"] == pytest.approx(ghz)
    assert k["mfma_busy"] == pytest.approx(busy)
    # busy MFMA pipes at the measured clock = the same fraction of that peak
    assert k["frac_peak_at_clock"] == pytest.approx(busy)
    assert k["frac_peak"] == pytest.approx(busy * ghz / 2.4)
    assert k["mfma_TFLOPs"] == pytest.approx(busy * 1024 * 1024 * ghz * 1e9 / 1e12)


def test_build_module_loads_without_the_package():
    """build() must work on a fresh checkout, where libfll.so does not exist
    yet and importing the package raises: it loads build.py by path."""
    code = (
        "import importlib.util, sys\n"
        f"spec = importlib.util.spec_from_file_location('_b', {os.path.join(ROOT, 'lm_head_projection_token_amd', 'build.py')!r})\n"
        "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
        "assert callable(m.build)\n"
        "assert 'lm_head_projection_token_amd' not in sys.modules\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=60)
    assert res.returncode == 0, res.stderr
    entry = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    assert "spec_from_file_location" in entry


def test_cpu_baseline_reports_the_oracle_on_a_row_sample():
    case = workloads.small_case(BT=64, H=32, V=100, head="selective", reduction="mean",
                                ignore_frac=0.1, seed=7)
    inp = workloads.make_inputs(case)
    out = bench.cpu_baseline(inp, case, rows_small=8, rows_big=32)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "extrapolated linearly to BT=64" in out["sample"]


@pytest.mark.gpu
def test_bench_json_line_on_the_gpu():
    """The benchmark's one JSON line: the fields the contract names, the
    roofline of the dominant GEMM and the per-kernel times (the V=32000 KL
    workload, a few steps)."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "2",
                          "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-clock"],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] == pytest.approx(1024 / (d["ms_per_step"] / 1e3), rel=1e-6)
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert 0.0 < r["frac"] < 1.0
    assert {"logits", "row", "dx", "prep", "final"} <= set(d["kernels"])


def test_clock_record_discards_impossible_readings():
    case = workloads.WORKLOADS[3]
    ms = 13.0
    # 1300 TFLOP/s needs at least 1300/2500*2.4 = 1.25 GHz
    ok = bench.clock_record((1.8, 1.7, 1.9, 6), case, ms, 1300.0)
    assert ok["GHz"] == 1.8
    assert ok["roofline_frac_at_clock"] == pytest.approx(1300.0 / (bench.PEAK_BF16_TFLOPS * 0.75))
    assert 0 < ok["end_to_end_frac_at_clock"] < 1
    bad = bench.clock_record((0.2, 0.2, 0.2, 6), case, ms, 1300.0)
    assert bad["GHz"] is None and bad["discarded_GHz"] == 0.2
    assert "roofline_frac_at_clock" not in bad


def test_clock_record_gives_no_fraction_for_identical_readings():
    # readings that repeat to the kHz are a stale amd-smi figure
    case = workloads.WORKLOADS[3]
    stale = bench.clock_record((2.2295, 2.2295, 2.2295, 6), case, 13.0, 1300.0)
    assert stale["GHz"] == 2.2295 and "stale" in stale["note"]
    assert "roofline_frac_at_clock" not in stale and "end_to_end_frac_at_clock" not in stale
    one = bench.clock_record((1.8, 1.8, 1.8, 1), case, 13.0, 1300.0)
    assert "roofline_frac_at_clock" in one


def test_measured_clock_needs_matching_sources(tmp_path, monkeypatch):
    from lm_head_projection_token_amd import profiling

    case = workloads.WORKLOADS[3]
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"src_sha256": profiling.source_hash(),
           "kernels": {"logits": {"clock_GHz": 1.82, "mfma_busy": 0.69}}}
    (prof / f"mfma_{case.name}.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_clock(case, "logits") == (1.82, 0.69)
    assert bench.measured_clock(case, "dx") is None
    rec["src_sha256"] = "0" * 64
    (prof / f"mfma_{case.name}.json").write_text(json.dumps(rec))
    assert bench.measured_clock(case, "logits") is None


def test_cpu_model_is_named():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_lds_summary_per_cu_and_conflict_share(tmp_path):
    d = tmp_path / "l"
    d.mkdir()
    rows = []
    for did, scale in ((3, 1.0), (7, 1.2), (11, 0.8)):
        for name, val in (("SQ_INSTS_LDS", 1000.0 * 256), ("SQ_LDS_IDX_ACTIVE", 4000.0 * 256),
                          ("SQ_LDS_BANK_CONFLICT", 40.0 * 256)):
            # each counter split over two instances of the dispatch
            for half in (0.5, 0.5):
                rows.append({"Dispatch_Id": did, "Kernel_Name": LOGITS, "Counter_Name": name,
                             "Counter_Value": val * scale * half})
    rows.append({"Dispatch_Id": 20, "Kernel_Name": ROW, "Counter_Name": "SQ_INSTS_LDS",
                 "Counter_Value": 5.0})
    _write_counters(d / "l_counter_collection.csv", rows)
    profiling.lds_summary(str(d), "x", "cmd", str(tmp_path / "lds_x"))
    rec = json.loads((tmp_path / "lds_x.json").read_text())["kernels"]
    k = rec["logits"]
    assert k["dispatches"] == 3
    assert k["lds_insts_per_cu"] == pytest.approx(1000.0)
    assert k["idx_active_per_cu"] == pytest.approx(4000.0)
    assert k["conflict_frac"] == pytest.approx(0.01)
    assert "row" not in rec  # a dispatch without every counter is left out
    assert "| logits | 3 |" in (tmp_path / "lds_x.md").read_text()


def test_ta_summary_busy_fraction(tmp_path):
    d = tmp_path / "a"
    d.mkdir()
    rows = []
    for did in (2, 4):
        for name, val in (("GRBM_GUI_ACTIVE", 8 * 1000.0), ("TA_BUSY_avr", 450.0),
                          ("TA_BUFFER_TOTAL_CYCLES_sum", 0.8 * 450.0 * 256)):
            rows.append({"Dispatch_Id": did, "Kernel_Name": LOGITS, "Counter_Name": name,
                         "Counter_Value": val})
    _write_counters(d / "a_counter_collection.csv", rows)
    profiling.ta_summary(str(d), "x", "cmd", str(tmp_path / "ta_x"))
    k = json.loads((tmp_path / "ta_x.json").read_text())["kernels"]["logits"]
    assert k["ta_busy_frac"] == pytest.approx(0.45)
    assert k["buffer_share"] == pytest.approx(0.8)
    assert k["dispatches"] == 2
