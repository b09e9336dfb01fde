"""The largest problems the ABI accepts, each in the dimension it stresses.

* V = 2^21 - 64, the largest vocabulary: 16384 statistics tiles per row,
  16 dX vocabulary splits, and a bf16 dZ row pitch of 2^22 elements, so a
  256-row dX operand tile spans just under the 2^31 bytes a buffer
  descriptor addresses. BT = 300 gives one full 256-row chunk and a ragged
  one. Checked against the oracle on sampled rows (per-row terms, dX) and by
  the properties that hold at any size (the loss reduction, <dX, X> =
  <dW, W>, zero column sums of dW and db).
* H = 2^20, the largest hidden size: a 32768-step K loop in the logits GEMM
  and 4096 output tiles across H in dX and dW. V is small, so the oracle
  runs in full.
* BT = 70001 tokens: the chunk size at its 8192-row cap, nine chunks with a
  ragged last one, dW and db accumulated over all of them; oracle in full.
All with a trainable head and a bias, in bf16 at the stated tolerances.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import fll_oracle
from tests import helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

V_MAX = (1 << 21) - 64
H_MAX = 1 << 20


def test_largest_vocabulary():
    case = workloads.small_case(BT=300, H=64, V=V_MAX, dtype="bf16", head="selective",
                                has_bias=True, compute_dW=True, compute_db=True,
                                reduction="mean", ignore_frac=0.05, w_std=0.05, seed=31)
    print(f"[limits] V = {V_MAX}: {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    plan = out["plan"]
    assert plan.dx_splits == 16 and plan.stat_tiles == -(-V_MAX // 128)
    labels = inp["labels"]
    rows = workloads.row_sample(case.BT, 16, seed=131, labels=labels)
    n_valid = int((labels != case.ignore_index).sum())
    ref = fll_oracle.sampled_rows(
        H.to_np(inp["X"][rows]), H.to_np(inp["W"]), H.to_np(inp["b"]), head=case.head,
        n_valid=n_valid, labels_rows=labels[rows].numpy(),
        weights_rows=H.to_np(inp["weights"][rows]), reduction=case.reduction,
        ignore_index=case.ignore_index, temperature=case.temperature, eps=case.eps)
    per = out["per_row"].cpu().double().numpy()
    scale = float(np.abs(ref["per_row"]).max())
    np.testing.assert_allclose(per[rows.numpy()], ref["per_row"], rtol=2e-3,
                               atol=2e-3 * scale, err_msg="per_row (sampled)")
    dX = out["dX"].float().cpu().double()
    H.check_grad(dX[rows].numpy(), ref["dX"], case.dtype, "dX (sampled rows)")
    w = inp["weights"].double().numpy()
    H.check_loss(float(out["loss"]), ref["g"] * float((w * per).sum()), "fp32",
                 "loss vs g * sum w * per_row")
    assert torch.count_nonzero(dX[labels == case.ignore_index]).item() == 0

    dW = out["dW"].cpu().double()
    X, W = inp["X"].double(), inp["W"].double()
    lhs, rhs = float((dX * X).sum()), float((dW * W).sum())
    assert abs(lhs - rhs) <= 1e-3 * float((dX.abs() * X.abs()).sum()), (lhs, rhs)
    col, colabs = dW.sum(dim=0).abs(), dW.abs().sum(dim=0)
    assert bool((col <= 1e-3 * colabs + 1e-12).all())
    db = out["db"].cpu().double()
    assert abs(float(db.sum())) <= 1e-3 * float(db.abs().sum())
    assert torch.isfinite(dW).all() and torch.isfinite(db).all()


def test_largest_hidden_size():
    case = workloads.small_case(BT=300, H=H_MAX, V=300, dtype="bf16", head="kl",
                                has_bias=True, compute_dW=True, compute_db=True,
                                temperature=2.0, ignore_frac=0.1, w_std=0.001, seed=32)
    print(f"[limits] H = {H_MAX}: {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    H.compare_full(out, H.run_oracle(inp, case), case)


@pytest.mark.parametrize("head", ["selective", "kl"])
def test_many_chunks_at_the_chunk_cap(head):
    # BT = 70001: the chunk size reaches its cap of 8192 rows, so the batch
    # runs in 9 chunks, the last one ragged (4465 rows); dW and db are
    # accumulated in fp32 over all of them. Oracle in full.
    case = workloads.small_case(BT=70001, H=64, V=1000, dtype="bf16", head=head,
                                has_bias=True, compute_dW=True, compute_db=True,
                                reduction="mean", ignore_frac=0.05, w_std=0.05, seed=33)
    print(f"[limits] BT = {case.BT}: {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    plan = out["plan"]
    assert plan.chunk_rows == 8192 and plan.n_chunks == 9
    H.compare_full(out, H.run_oracle(inp, case), case, inp=inp)
