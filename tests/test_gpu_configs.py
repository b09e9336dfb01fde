"""The five named workloads at full size, in the launch configuration the
benchmark times (the default plan).

cfg1 (tiny fp32) and cfg2 (V = 32000) are compared with the oracle element
by element. cfg3-cfg5 are too large for the oracle to form every logit in
seconds, so they are checked on sampled token rows -- the per-row loss terms
and dX rows, which the oracle computes row by row with the global valid-row
count -- and by properties that hold at any size:
  * the loss is g * sum_r w_r * per_row_r (the reduction step);
  * <dX, X> = <dW, W> (both equal sum_{r,v} dZ_rv Z'_rv with Z' = X W^T);
  * every dlogits row sums to zero, so each column of dW sums to zero over
    the vocabulary and db sums to zero;
  * ignored rows have exactly zero dX.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import fll_oracle
from tests import helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_cfg1_full():
    case = workloads.WORKLOADS[1]
    inp = H.make(case)
    H.compare_full(H.run_gpu(inp, case), H.run_oracle(inp, case), case)


def test_cfg2_full():
    case = workloads.WORKLOADS[2]
    print(f"[cfg2] {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    ref = H.run_oracle(inp, case)
    H.compare_full(out, ref, case)


# The fused linear cross-entropy head at the llama-3 head shape of the
# V=128256 GRPO workload, with a trainable head (beyond the five workloads).
CE_FULL = workloads.WORKLOADS[3].replace(name="ce-bf16-trainable-B8T1024-V128256", head="ce",
                                       compute_dW=True, ignore_frac=0.05, seed=6)
EXTRA = {"ce": CE_FULL, "jsd": workloads.JSD_WORKLOAD}


# "-bf16-logits": the same workload with the chunk logits kept in bf16
@pytest.mark.parametrize("cfg", [3, 4, 5, "ce", "jsd", "3-bf16-logits", "5-bf16-logits",
                                 "jsd-bf16-logits"])
def test_full_config_sampled(cfg):
    logits_bf16 = isinstance(cfg, str) and cfg.endswith("-bf16-logits")
    key = cfg[:-len("-bf16-logits")] if logits_bf16 else cfg
    key = int(key) if isinstance(key, str) and key.isdigit() else key
    case = EXTRA[key] if key in EXTRA else workloads.WORKLOADS[key]
    print(f"[cfg{cfg}] {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case, logits_bf16=logits_bf16)
    labels = inp["labels"]
    rows = workloads.row_sample(case.BT, 24, seed=100 + case.seed, labels=labels)
    n_valid = case.BT if labels is None else int((labels != case.ignore_index).sum())
    ref = fll_oracle.sampled_rows(
        H.to_np(inp["X"][rows]), H.to_np(inp["W"]), H.to_np(inp["b"]), head=case.head,
        n_valid=n_valid,
        labels_rows=None if labels is None else labels[rows].numpy(),
        target_rows=None if inp["target"] is None else H.to_np(inp["target"][rows]),
        weights_rows=None if inp["weights"] is None else H.to_np(inp["weights"][rows]),
        reduction=case.reduction, ignore_index=case.ignore_index,
        temperature=case.temperature, eps=case.eps,
        Xt_rows=None if inp["X_teacher"] is None else H.to_np(inp["X_teacher"][rows]),
        W_teacher=H.to_np(inp["W_teacher"]), b_teacher=H.to_np(inp["b_teacher"]))
    print(f"[cfg{cfg}] oracle rows done", flush=True)

    per = out["per_row"].cpu().double().numpy()
    scale = float(np.abs(ref["per_row"]).max())
    atol = 2e-3 * scale
    # plus what rounding the logits to bf16 can move a row's term; the label
    # heads take the label's logit in fp32 from the GEMM, so theirs do not move
    if logits_bf16 and case.head not in ("selective", "ce"):
        atol = atol + H.logit_rounding_bound(inp, case, rows)
    err = np.abs(per[rows.numpy()] - ref["per_row"])
    assert (err <= atol + 2e-3 * np.abs(ref["per_row"])).all(), \
        f"per_row (sampled): max err {err.max():.3e}"
    dX = out["dX"].float().cpu()
    H.check_grad(dX[rows].double().numpy(), ref["dX"], case.dtype, "dX (sampled rows)")

    # the loss is the reduction of the per-row terms
    w = np.ones(case.BT) if inp["weights"] is None else inp["weights"].double().numpy()
    g = ref["g"]
    H.check_loss(float(out["loss"]), g * float((w * per).sum()), "fp32",
                 "loss vs g * sum w * per_row")
    assert np.isfinite(per).all()

    if labels is not None:
        ign = (labels == case.ignore_index)
        if bool(ign.any()):
            assert torch.count_nonzero(dX[ign]).item() == 0

    if case.compute_dW:
        dW = out["dW"].cpu().double()
        W = inp["W"].double()
        X = inp["X"].double()
        lhs = float((dX.double() * X).sum())
        rhs = float((dW * W).sum())
        bound = float((dX.double().abs() * X.abs()).sum())
        assert abs(lhs - rhs) <= 1e-3 * bound, (lhs, rhs, bound)
        col = dW.sum(dim=0).abs()
        colabs = dW.abs().sum(dim=0)
        assert bool((col <= 1e-3 * colabs + 1e-12).all()), float((col / colabs).max())
        assert torch.isfinite(dW).all()
    if case.compute_db:
        db = out["db"].cpu().double()
        assert abs(float(db.sum())) <= 1e-3 * float(db.abs().sum())
        assert torch.isfinite(db).all()
