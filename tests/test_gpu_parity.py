"""Parity of the HIP path with the CPU oracle, element by element.

Sizes are chosen so the oracle finishes in seconds while the GPU kernels
still run several 256 x 256 tiles with ragged tails in every dimension:
H = 264 and 136 are not multiples of the 64-wide K-step or the 256-wide
tile, V = 1000 / 777 / 4099 leave partial vocabulary tiles (777 is odd, so
rows are not 16-byte multiples), and BT = 300 / 520 leave a partial last
token chunk.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from tests import helpers as H

pytestmark = pytest.mark.gpu

SMALL = {
    "cfg1-tiny-fp32-kl": workloads.WORKLOADS[1],
    "kl-bf16-ragged-trainable-bias": workloads.small_case(
        BT=300, H=264, V=1000, dtype="bf16", head="kl", has_bias=True, compute_dW=True,
        compute_db=True, temperature=2.0, ignore_frac=0.1, reduction="batchmean",
        x_std=1.0, w_std=0.05, seed=11),
    "sel-bf16-odd-vocab-trainable": workloads.small_case(
        BT=520, H=136, V=777, dtype="bf16", head="selective", has_bias=True,
        compute_dW=True, compute_db=True, reduction="mean", ignore_frac=0.05,
        w_std=0.05, seed=12),
    "sel-bf16-frozen-sum-two-vocab-chunks": workloads.small_case(
        BT=300, H=256, V=4099, dtype="bf16", head="selective", reduction="sum",
        temperature=0.5, w_std=0.02, seed=13),
    "kl-bf16-mean-no-labels": workloads.small_case(
        BT=257, H=64, V=2048, dtype="bf16", head="kl", reduction="mean", with_labels=False,
        compute_dW=True, w_std=0.05, seed=14),
    "sel-fp32-trainable": workloads.small_case(
        BT=130, H=72, V=333, dtype="fp32", head="selective", has_bias=True,
        compute_dW=True, compute_db=True, reduction="batchmean", x_std=1.0, w_std=0.1,
        seed=15),
    "ce-bf16-ragged-trainable-bias": workloads.small_case(
        BT=300, H=264, V=1000, dtype="bf16", head="ce", has_bias=True, compute_dW=True,
        compute_db=True, reduction="mean", ignore_frac=0.1, w_std=0.05, seed=17),
    "ce-fp32-sum-tau": workloads.small_case(
        BT=90, H=48, V=301, dtype="fp32", head="ce", compute_dW=True, reduction="sum",
        temperature=0.5, x_std=1.0, w_std=0.1, seed=18),
    # Jensen-Shannon head: the teacher has its own projection of another
    # hidden size (and a bias), the student a ragged vocabulary
    "jsd-bf16-ragged-trainable-teacher-bias": workloads.small_case(
        BT=300, H=264, V=1000, dtype="bf16", head="jsd", has_bias=True, compute_dW=True,
        compute_db=True, H_teacher=136, teacher_has_bias=True, teacher_w_std=0.05,
        temperature=2.0, ignore_frac=0.1, reduction="batchmean", w_std=0.05, seed=19),
    "jsd-bf16-mean-odd-vocab": workloads.small_case(
        BT=257, H=64, V=777, dtype="bf16", head="jsd", H_teacher=264, reduction="mean",
        with_labels=False, w_std=0.1, teacher_w_std=0.1, seed=20),
    "jsd-fp32-sum-tau": workloads.small_case(
        BT=90, H=48, V=301, dtype="fp32", head="jsd", compute_dW=True, H_teacher=40,
        reduction="sum", temperature=0.5, ignore_frac=0.2, x_std=1.0, w_std=0.1,
        teacher_w_std=0.1, seed=21),
    "kl-fp32-sum-ignored": workloads.small_case(
        BT=100, H=40, V=515, dtype="fp32", head="kl", reduction="sum", ignore_frac=0.2,
        compute_dW=True, x_std=1.0, w_std=0.1, temperature=0.75, seed=16),
    # ratio heads (old log-probs = the oracle's log p(y) minus drawn
    # log-ratios, kept off the clip edges): DAPO's wider upper clip, both
    # clip branches, ragged shapes
    "ppo-bf16-ragged-trainable-bias": workloads.small_case(
        BT=300, H=264, V=1000, dtype="bf16", head="ppo", has_bias=True, compute_dW=True,
        compute_db=True, clip_low=0.2, clip_high=0.28, logratio_std=0.4, temperature=2.0,
        ignore_frac=0.1, reduction="mean", w_std=0.05, seed=41),
    "cispo-bf16-odd-vocab-sum": workloads.small_case(
        BT=520, H=136, V=777, dtype="bf16", head="cispo", compute_dW=True,
        clip_low=0.2, clip_high=0.28, logratio_std=0.4, reduction="sum", ignore_frac=0.05,
        w_std=0.05, seed=42),
    "ppo-fp32-trainable": workloads.small_case(
        BT=130, H=72, V=333, dtype="fp32", head="ppo", has_bias=True, compute_dW=True,
        compute_db=True, clip_low=0.1, clip_high=0.1, logratio_std=0.3, x_std=1.0,
        w_std=0.1, seed=43),
    # db with a frozen weight (the column-sum kernel; with dW, db is formed
    # inside the dW GEMM), a vocabulary tail in the last 256-row tile
    "sel-bf16-db-only-frozen-weight": workloads.small_case(
        BT=520, H=136, V=1100, dtype="bf16", head="selective", has_bias=True,
        compute_db=True, reduction="sum", ignore_frac=0.05, w_std=0.05, seed=46),
    # a ragged last chunk (44 tokens) with the dX vocabulary split (4
    # splits), a trainable head and bias: the transposed X of the dW GEMM
    # shares its buffer with the dX partial sums
    "sel-bf16-ragged-chunk-split-dx-trainable": workloads.small_case(
        BT=300, H=136, V=8192, dtype="bf16", head="selective", has_bias=True,
        compute_dW=True, compute_db=True, reduction="mean", ignore_frac=0.05,
        w_std=0.05, seed=47),
    "ppo-bf16-no-clip-two-vocab-chunks": workloads.small_case(
        BT=257, H=64, V=4099, dtype="bf16", head="ppo", clip_low=1.0,
        clip_high=float("inf"), logratio_std=0.5, reduction="mean", w_std=0.05, seed=44),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_parity(name):
    case = SMALL[name]
    print(f"[parity] {name} {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    ref = H.run_oracle(inp, case)
    H.compare_full(out, ref, case)


BF16_SMALL = sorted(k for k, c in SMALL.items() if c.dtype == "bf16")


@pytest.mark.parametrize("name", BF16_SMALL)
def test_small_parity_bf16_logits(name):
    # chunk logits kept in bf16: the same cases and the same loss and gradient
    # tolerances; the per-row terms of the KL and JSD heads also allow for the
    # logits' rounding (the label heads take the label's logit in fp32 from
    # the logits GEMM and the log-sum-exp from its fp32 statistics)
    case = SMALL[name]
    print(f"[parity bf16 logits] {name} {case}", flush=True)
    inp = H.make(case)
    extra = 0.0 if case.head in workloads.LABEL_HEADS else H.logit_rounding_bound(inp, case)
    H.compare_full(H.run_gpu(inp, case, logits_bf16=True), H.run_oracle(inp, case), case,
                   per_row_atol=extra)


@pytest.mark.parametrize("head", ["kl", "selective", "jsd"])
def test_bf16_logits_dx_independent_of_gradient_flags(head):
    # with bf16 chunk logits too, dX does not depend on compute_dW / compute_db
    kw = dict(H_teacher=72) if head == "jsd" else {}
    case = workloads.small_case(BT=600, H=136, V=1500, dtype="bf16", head=head,
                                has_bias=True, ignore_frac=0.1, w_std=0.05, seed=23, **kw)
    inp = H.make(case)
    a = H.run_gpu(inp, case, logits_bf16=True)
    b = H.run_gpu(inp, case.replace(compute_dW=True, compute_db=True), logits_bf16=True)
    assert torch.equal(a["dX"], b["dX"])
    assert torch.equal(a["loss"], b["loss"])


@pytest.mark.parametrize("eps", [0.0, 1e-10])
def test_kl_one_hot_targets(eps):
    # exact zeros in every target row: each contributes 0 to the KL (for
    # eps = 0 too), which is then the cross-entropy (FusedLinearKLDivLoss
    # page, Details: 0 log 0 contributes 0)
    case = workloads.small_case(BT=300, H=264, V=1000, dtype="bf16", head="kl",
                                has_bias=True, compute_dW=True, compute_db=True,
                                temperature=2.0, ignore_frac=0.1, w_std=0.05, eps=eps,
                                seed=45)
    inp = H.make(case)
    keep = inp["labels"] != case.ignore_index
    q = torch.zeros_like(inp["target"])
    q[keep, inp["labels"][keep]] = 1.0
    q[~keep] = float("nan")
    inp["target"] = q
    out = H.run_gpu(inp, case)
    assert torch.isfinite(out["per_row"]).all() and torch.isfinite(out["loss"])
    H.compare_full(out, H.run_oracle(inp, case), case)
    ce = H.run_gpu(dict(inp, target=None), case.replace(head="ce", with_weights=False))
    torch.testing.assert_close(out["per_row"], ce["per_row"], rtol=2e-3, atol=2e-3)


def test_ratio_clip_branches_on_the_gpu():
    # the rows the oracle takes as clipped get exactly zero dlogits (dX row
    # 0), the others not: the clip decision is the oracle's on every row
    case = SMALL["ppo-bf16-ragged-trainable-bias"]
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    d = inp["logratio"].double()
    old = H.ratio_old_logprobs(inp, case)
    keep = inp["labels"] != case.ignore_index
    A = inp["weights"].double()
    rho = d.exp()
    c = rho.clamp(1 - case.clip_low, 1 + case.clip_high)
    clipped = keep & (rho * A > c * A)
    assert 0 < int(clipped.sum()) < int(keep.sum())
    zero_rows = (out["dX"].cpu() == 0).all(dim=1)
    assert torch.equal(zero_rows, clipped | ~keep), (zero_rows ^ (clipped | ~keep)).nonzero()
    assert torch.isfinite(old[keep]).all()


@pytest.mark.parametrize("head", ["ppo", "cispo"])
def test_ratio_heads_at_ratio_one_match_the_selective_head(head):
    # old = the oracle's log p(y): every ratio is one (up to fp32 rounding of
    # the input), so dX equals the selective head's with weights -A
    case = SMALL["ppo-bf16-ragged-trainable-bias"].replace(head=head)
    inp = H.make(case)
    inp["logratio"] = torch.zeros_like(inp["logratio"])
    out = H.run_gpu(inp, case)
    sel_case = case.replace(head="selective")
    sel_inp = dict(inp, weights=-inp["weights"])
    sel = H.run_gpu(sel_inp, sel_case)
    torch.testing.assert_close(out["dX"].float(), sel["dX"].float(), rtol=2e-2,
                               atol=1e-2 * float(sel["dX"].float().abs().max()))
    H.check_grad(out["dW"].cpu().numpy(), sel["dW"].cpu().numpy(), "bf16", "dW vs selective")


def test_unnormalised_target():
    # target rows summing to 1.3: the exact gradient uses Q_r = sum_v q_rv
    case = workloads.small_case(BT=96, H=64, V=300, dtype="fp32", head="kl",
                                compute_dW=True, reduction="batchmean", x_std=1.0,
                                w_std=0.1, seed=21)
    inp = H.make(case)
    inp["target"] = inp["target"] * 1.3
    H.compare_full(H.run_gpu(inp, case), H.run_oracle(inp, case), case)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("head", ["selective", "kl", "ce", "jsd", "ppo", "cispo"])
def test_all_rows_ignored(dtype, head):
    extra = dict(H_teacher=24) if head == "jsd" else {}
    case = workloads.small_case(BT=64, H=32, V=100, dtype=dtype, head=head,
                                has_bias=True, compute_dW=True, compute_db=True, seed=22,
                                **extra)
    inp = H.make(case)
    inp["labels"][:] = case.ignore_index
    if inp["target"] is not None:
        inp["target"][:] = float("nan")  # ignored rows' targets are never read
    out = H.run_gpu(inp, case)
    assert float(out["loss"]) == 0.0
    for k in ("dX", "dW", "db", "per_row"):
        assert torch.count_nonzero(out[k]).item() == 0, k


@pytest.mark.parametrize("head", ["kl", "selective", "jsd", "ce", "ppo", "cispo"])
def test_empty_batch(head):
    import lm_head_projection_token_amd as fll

    dev = "cuda:0"
    X = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    W = torch.randn(50, 64, device=dev).to(torch.bfloat16)
    b = torch.zeros(50, dtype=torch.bfloat16, device=dev)
    kw = dict(labels=torch.empty(0, dtype=torch.int64, device=dev))
    if head == "kl":
        kw["target"] = torch.empty(0, 50, device=dev)
    if head == "jsd":
        kw["X_teacher"] = torch.empty(0, 32, dtype=torch.bfloat16, device=dev)
        kw["W_teacher"] = torch.randn(50, 32, device=dev).to(torch.bfloat16)
    if head in ("ppo", "cispo"):
        kw["old_logprobs"] = torch.empty(0, device=dev)
    out = fll.fused_lm_head_loss(X, W, b, head=head, compute_dW=True, compute_db=True, **kw)
    torch.cuda.synchronize()
    assert float(out["loss"]) == 0.0
    assert out["dX"].shape == (0, 64)
    assert torch.count_nonzero(out["dW"]).item() == 0
    assert torch.count_nonzero(out["db"]).item() == 0


@pytest.mark.parametrize("head", ["kl", "selective", "jsd", "ce", "ppo", "cispo"])
def test_single_token_vocabulary(head):
    # V = 1: log p = 0 for every row, so every gradient vanishes exactly (the
    # block statistics give the row maximum exactly 1, so p = 1); the loss
    # is 0 too, except for the ratio heads, whose terms depend on the old
    # log-probs and advantages only.
    extra = dict(H_teacher=24) if head == "jsd" else {}
    case = workloads.small_case(BT=40, H=16, V=1, dtype="bf16", head=head,
                                compute_dW=True, seed=23, **extra)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    ref = H.run_oracle(inp, case)
    assert abs(float(out["loss"]) - ref["loss"]) <= 1e-6
    assert torch.count_nonzero(out["dX"]).item() == 0


@pytest.mark.parametrize("head", ["selective", "ce", "ppo", "cispo"])
def test_out_of_range_label_is_nan_not_a_fault(head):
    case = workloads.small_case(BT=64, H=32, V=100, dtype="bf16", head=head,
                                compute_dW=True, seed=24)
    inp = H.make(case)
    if head in workloads.RATIO_HEADS:
        H.ratio_old_logprobs(inp, case)  # from the in-range labels
    inp["labels"][5] = 100   # == V
    inp["labels"][9] = -7    # negative, not ignore_index
    out = H.run_gpu(inp, case)
    assert np.isnan(float(out["loss"]))
    per = out["per_row"].cpu()
    assert torch.isnan(per[5]) and torch.isnan(per[9])
    assert torch.count_nonzero(out["dX"][5]).item() == 0
    assert torch.isfinite(out["dX"]).all() and torch.isfinite(out["dW"]).all()


# --------------------------------------------------------------------------
# bit-identity and determinism
# --------------------------------------------------------------------------

BITCASE = workloads.small_case(BT=600, H=136, V=1000, dtype="bf16", head="kl",
                               has_bias=True, compute_dW=True, compute_db=True,
                               temperature=2.0, ignore_frac=0.1, w_std=0.05, seed=31)


def test_dx_bit_identical_frozen_vs_trainable():
    # LoRA normalization page, Test Validation: the input gradient is exactly
    # equal whether or not the weight gradients are formed.
    inp = H.make(BITCASE)
    trainable = H.run_gpu(inp, BITCASE)
    frozen_case = BITCASE.replace(compute_dW=False, compute_db=False)
    frozen = H.run_gpu(inp, frozen_case)
    assert torch.equal(trainable["dX"], frozen["dX"])
    assert torch.equal(trainable["loss"], frozen["loss"])
    assert frozen["dW"] is None and frozen["db"] is None


def test_frozen_head_leaves_dw_untouched():
    # With compute_dW = compute_db = 0 the call may be handed dW / db buffers
    # and must not touch them [frozen lm_head GRPO page, Summary].
    import lm_head_projection_token_amd as fll

    case = BITCASE.replace(compute_dW=False, compute_db=False)
    inp = H.make(case)
    dev = "cuda:0"
    X, W, b = (inp[k].to(dev) for k in ("X", "W", "b"))
    prob = fll.make_problem(case.BT, case.H, case.V, dtype="bf16", head="kl", has_bias=True,
                            temperature=case.temperature)
    plan = fll.fll_plan(prob)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    dW = torch.full((case.V, case.H), 7.25, device=dev)
    db = torch.full((case.V,), -3.5, device=dev)
    loss = torch.empty((), device=dev)
    dX = torch.empty_like(X)
    fll.fll_fwd_bwd(plan, X=X, W=W, b=b, labels=inp["labels"].to(dev),
                    target=inp["target"].to(dev), dX=dX, dW=dW, db=db, loss=loss,
                    workspace=ws)
    torch.cuda.synchronize()
    assert bool((dW == 7.25).all()) and bool((db == -3.5).all())
    assert torch.isfinite(dX).all() and torch.isfinite(loss)


def test_chunk_size_does_not_change_dx():
    # V < 2048: the dX GEMM never splits the vocabulary, so every dX row is
    # summed in the same order whatever the chunk size
    inp = H.make(BITCASE)
    base = H.run_gpu(inp, BITCASE)
    assert base["plan"].n_chunks >= 2
    for C in (100, 37, 600):
        other = H.run_gpu(inp, BITCASE, chunk_rows=C)
        assert other["plan"].chunk_rows == C
        assert torch.equal(base["dX"], other["dX"]), C
        assert torch.equal(base["per_row"], other["per_row"]), C
        # dW / db are sums over chunks: equal up to fp32 reassociation
        torch.testing.assert_close(other["dW"], base["dW"], rtol=1e-5,
                                   atol=1e-6 * float(base["dW"].abs().max()))
        torch.testing.assert_close(other["db"], base["db"], rtol=1e-5,
                                   atol=1e-6 * float(base["db"].abs().max()))


def test_chunk_size_changes_dx_only_by_reassociation():
    # the vocabulary split of dX follows the chunk size (one workgroup per CU:
    # 8 splits at C = 512, 6 at C = 768, 4 at C = 1024 here), so dX rows are
    # fp32 sums in another order: equal to a bf16 rounding step; the per-row
    # loss terms do not depend on it
    case = workloads.small_case(BT=1024, H=4096, V=32768, dtype="bf16", head="selective",
                                compute_dW=True, seed=35)
    inp = H.make(case)
    base = H.run_gpu(inp, case)
    splits = {base["plan"].dx_splits}
    for C in (768, 1024):
        other = H.run_gpu(inp, case, chunk_rows=C)
        splits.add(other["plan"].dx_splits)
        assert torch.equal(base["per_row"], other["per_row"]), C
        assert torch.equal(base["loss"], other["loss"]), C
        torch.testing.assert_close(other["dX"].float(), base["dX"].float(), rtol=2 ** -7,
                                   atol=1e-3 * float(base["dX"].float().abs().max()))
        torch.testing.assert_close(other["dW"], base["dW"], rtol=1e-5,
                                   atol=1e-6 * float(base["dW"].abs().max()))
    assert len(splits) > 1, splits


@pytest.mark.parametrize("head", ["kl", "selective", "ce", "jsd", "ppo", "cispo"])
def test_repeated_calls_are_bitwise_equal(head):
    # no atomics and fixed-order reductions: every output repeats bit for bit
    # (V = 8192 also splits the dX vocabulary range)
    extra = dict(H_teacher=72) if head == "jsd" else {}
    case = BITCASE if head == "kl" else BITCASE.replace(head=head, V=8192, **extra)
    inp = H.make(case)
    a = H.run_gpu(inp, case)
    b = H.run_gpu(inp, case)
    for k in ("loss", "dX", "dW", "db", "per_row"):
        assert torch.equal(a[k], b[k]), k


def test_temperature_power_of_two_identity():
    # (X W^T + b) / 2 == X (W / 2)^T + b / 2 exactly in the GEMM's fp32
    # accumulation, so dX agrees bitwise and dW(tau) = dW'(1) / tau.
    case = workloads.small_case(BT=300, H=136, V=1000, dtype="bf16", head="selective",
                                has_bias=True, compute_dW=True, compute_db=True,
                                temperature=2.0, w_std=0.05, seed=32)
    inp = H.make(case)
    a = H.run_gpu(inp, case)
    inp2 = dict(inp)
    inp2["W"] = (inp["W"].float() / 2).to(torch.bfloat16)
    inp2["b"] = (inp["b"].float() / 2).to(torch.bfloat16)
    b = H.run_gpu(inp2, case.replace(temperature=1.0))
    assert torch.equal(a["loss"], b["loss"])
    torch.testing.assert_close(a["dX"].float(), b["dX"].float(), rtol=0, atol=0)
    torch.testing.assert_close(a["dW"], b["dW"] / 2, rtol=0, atol=0)


def test_ce_per_token_weights():
    case = workloads.small_case(BT=200, H=64, V=513, dtype="fp32", head="ce",
                                compute_dW=True, reduction="mean", x_std=1.0,
                                w_std=0.1, seed=25)
    inp = H.make(case)
    inp["weights"] = torch.rand(case.BT, generator=torch.Generator().manual_seed(7))
    H.compare_full(H.run_gpu(inp, case), H.run_oracle(inp, case), case)


# --------------------------------------------------------------------------
# Jensen-Shannon head
# --------------------------------------------------------------------------

def test_jsd_teacher_equal_to_student_gives_zero():
    # the same projection on both sides: both logits GEMMs produce identical
    # rows, every log-ratio is exactly 0, so the loss and every gradient are 0
    case = workloads.small_case(BT=300, H=136, V=1000, dtype="bf16", head="jsd",
                                has_bias=True, compute_dW=True, compute_db=True,
                                H_teacher=136, teacher_has_bias=True, temperature=2.0,
                                w_std=0.05, seed=33)
    inp = H.make(case)
    inp["X_teacher"], inp["W_teacher"], inp["b_teacher"] = inp["X"], inp["W"], inp["b"]
    out = H.run_gpu(inp, case)
    assert float(out["loss"]) == 0.0
    for k in ("dX", "dW", "db", "per_row"):
        assert torch.count_nonzero(out[k]).item() == 0, k


def test_jsd_rows_within_bounds_and_dx_independent_of_flags():
    case = workloads.small_case(BT=520, H=136, V=4099, dtype="bf16", head="jsd",
                                H_teacher=264, compute_dW=True, ignore_frac=0.05,
                                w_std=0.2, teacher_w_std=0.2, seed=34)
    inp = H.make(case)
    a = H.run_gpu(inp, case)
    per = a["per_row"].cpu()
    assert bool((per >= 0).all()) and bool((per <= math.log(2) * (1 + 1e-5)).all())
    b = H.run_gpu(inp, case.replace(compute_dW=False))
    assert torch.equal(a["dX"], b["dX"]) and torch.equal(a["loss"], b["loss"])


# --------------------------------------------------------------------------
# HIP graph capture
# --------------------------------------------------------------------------

def test_graph_capture_replays_match_eager():
    # fll_fwd_bwd only launches kernels (zero fills are kernels too), so it
    # can be captured into a HIP graph; every replay, with eager work and
    # synchronisation in between, must reproduce the eager result bitwise
    import lm_head_projection_token_amd as fll

    case = workloads.small_case(BT=520, H=136, V=777, dtype="bf16", head="selective",
                                has_bias=True, compute_dW=True, compute_db=True,
                                reduction="mean", ignore_frac=0.05, w_std=0.05, seed=36)
    inp = H.make(case)
    dev = "cuda:0"
    X, W, b = (inp[k].to(dev) for k in ("X", "W", "b"))
    labels, weights = inp["labels"].to(dev), inp["weights"].to(dev)
    prob = fll.make_problem(case.BT, case.H, case.V, dtype="bf16", head="selective",
                            has_bias=True, compute_dW=True, compute_db=True, reduction="mean")
    plan = fll.fll_plan(prob)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    outs = dict(dX=torch.empty_like(X), dW=torch.empty(case.V, case.H, device=dev),
                db=torch.empty(case.V, device=dev), loss=torch.empty((), device=dev),
                per_row=torch.empty(case.BT, device=dev))

    def call(stream=None):
        fll.fll_fwd_bwd(plan, X=X, W=W, b=b, labels=labels, weights=weights, workspace=ws,
                        stream=stream, **outs)

    call()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    for v in outs.values():
        v.fill_(float("nan"))
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    for rep in range(3):
        for v in outs.values():
            v.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, eager[k]), (rep, k)


def test_concurrent_calls_on_two_streams_and_threads():
    # the library keeps no state between calls: two problems, each with its
    # own workspace, enqueued on two streams from two host threads at once,
    # give bitwise the results each gives alone
    import threading

    import lm_head_projection_token_amd as fll

    cases = [workloads.small_case(BT=520, H=136, V=1100, dtype="bf16", head="selective",
                                  has_bias=True, compute_dW=True, compute_db=True,
                                  reduction="mean", ignore_frac=0.05, w_std=0.05, seed=71),
             workloads.small_case(BT=300, H=264, V=1000, dtype="bf16", head="kl",
                                  compute_dW=True, temperature=2.0, ignore_frac=0.1,
                                  w_std=0.05, seed=72)]
    dev = "cuda:0"
    runs = []
    for case in cases:
        inp = H.make(case)
        d = {k: (None if inp.get(k) is None else inp[k].to(dev))
             for k in ("X", "W", "b", "labels", "target", "weights")}
        prob = fll.make_problem(case.BT, case.H, case.V, dtype="bf16", head=case.head,
                                has_bias=case.has_bias, compute_dW=case.compute_dW,
                                compute_db=case.compute_db, reduction=case.reduction,
                                temperature=case.temperature)
        plan = fll.fll_plan(prob)
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        outs = dict(dX=torch.empty_like(d["X"]), loss=torch.empty((), device=dev),
                    dW=torch.empty(case.V, case.H, device=dev),
                    db=torch.empty(case.V, device=dev) if case.compute_db else None)
        runs.append((plan, d, ws, outs))

    def call(run, stream=None):
        plan, d, ws, outs = run
        fll.fll_fwd_bwd(plan, **d, workspace=ws, stream=stream, **outs)

    alone = []
    for run in runs:
        call(run)
        torch.cuda.synchronize()
        alone.append({k: v.clone() for k, v in run[3].items() if v is not None})
        for v in run[3].values():
            if v is not None:
                v.fill_(float("nan"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(i):
        try:
            for _ in range(3):
                call(runs[i], streams[i])
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for run, ref in zip(runs, alone):
        for k, v in ref.items():
            assert torch.equal(run[3][k], v), k
