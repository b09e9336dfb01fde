"""The boundary from plain C: ``tests/c_client/fll_client.c`` includes
include/fll.h, links the in-tree libfll.so and the HIP runtime (gcc, no
Python, no torch), plans problems and runs fll_fwd_bwd on device memory of
its own. Host-only checks run without a GPU; the GPU case compares the C
client's outputs with the oracle at the stated tolerances."""

import os
import subprocess

import numpy as np
import pytest
import torch

import workloads
from tests import helpers as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "fll_client")


def client():
    if not os.path.exists(CLIENT):
        import importlib.util

        spec = importlib.util.spec_from_file_location(
            "_fll_build", os.path.join(ROOT, "lm_head_projection_token_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build_c_client()
    return CLIENT


def test_c_client_plans_and_gets_the_documented_errors():
    res = subprocess.run([client(), "plan"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"


def test_c_client_usage_error():
    res = subprocess.run([client()], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "usage" in res.stderr


def _write_inputs(d, inp, case):
    def raw(name, t):
        if t is None:
            return
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        t.numpy().tofile(os.path.join(d, name))

    raw("X.bin", inp["X"])
    raw("W.bin", inp["W"])
    raw("b.bin", inp["b"])
    raw("labels.bin", inp["labels"])
    raw("weights.bin", inp["weights"])
    red = {"batchmean": 0, "mean": 1, "sum": 2}[case.reduction]
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"{case.BT} {case.H} {case.V} {red} {int(case.has_bias)} "
                f"{int(case.compute_dW)} {int(case.compute_db)} {case.temperature!r} "
                f"{int(inp['weights'] is not None)} {case.ignore_index}\n")


def _read(d, name, dtype, shape):
    a = np.fromfile(os.path.join(d, name), dtype=dtype).reshape(shape)
    if dtype == np.int16:
        return torch.from_numpy(a.copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


@pytest.mark.gpu
def test_c_client_matches_the_oracle(tmp_path):
    case = workloads.small_case(BT=520, H=136, V=1100, dtype="bf16", head="selective",
                                has_bias=True, compute_dW=True, compute_db=True,
                                reduction="mean", temperature=2.0, ignore_frac=0.1,
                                w_std=0.05, seed=61)
    inp = H.make(case)
    d = str(tmp_path)
    _write_inputs(d, inp, case)
    print(f"[c client] {case}", flush=True)
    res = subprocess.run([client(), "run", d], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    out = dict(loss=_read(d, "loss.bin", np.float32, ())[()],
               per_row=_read(d, "per_row.bin", np.float32, (case.BT,)),
               dX=_read(d, "dX.bin", np.int16, (case.BT, case.H)),
               dW=_read(d, "dW.bin", np.float32, (case.V, case.H)),
               db=_read(d, "db.bin", np.float32, (case.V,)))
    H.compare_full(out, H.run_oracle(inp, case), case, inp=inp)
