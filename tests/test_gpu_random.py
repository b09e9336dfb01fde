"""Seeded random configurations against the oracle.

The hand-picked parity cases each fix one combination of head, dtype,
shape and options. Here every option is drawn together from a seeded
generator: head, dtype, token count, hidden size and vocabulary size
(ragged and degenerate values included: 1 token, a 1-entry vocabulary,
sizes one off a 256-wide tile), bias, gradient flags, reduction,
temperature, ignored rows, weights, forced chunk sizes that are not tile
multiples, and bf16 chunk logits. Each case is compared element by element
with the oracle at the stated tolerances; the per-row terms of the KL and
JSD heads with bf16 chunk logits also allow for the logits' rounding, every
per-row term a few float32 ulps of the row's largest logit (a one-entry
vocabulary has exact zeros that float32 reaches only to that), and a bf16
gradient element the rounding bound of the bf16 dlogits (sum reduction
gives gradients of order one, where the stated absolute tolerance is
finer than that rounding on elements that cancel).
"""

import numpy as np
import pytest

import lm_head_projection_token_amd as fll
import workloads
from tests import helpers as H

N_CASES = 40
HEADS = ("kl", "selective", "ce", "jsd", "ppo", "cispo")


def draw(i):
    """Case i of the sweep, with its forced chunk size (0: the planner's) and
    whether the chunk logits are bf16."""
    rng = np.random.default_rng(7000 + i)
    head = HEADS[i % len(HEADS)]  # every head equally often
    dtype = "fp32" if rng.random() < 0.2 else "bf16"
    BT = int(rng.choice([1, 2, 17, 64, 255, 256, 257, 300, 511, 640]))
    Hd = 8 * int(rng.integers(1, 41))
    V = int(rng.choice([1, 7, 100, 255, 256, 257, 777, 1000, 2049, 4099]))
    has_bias = bool(rng.random() < 0.5)
    compute_dW = bool(rng.random() < 0.5)
    compute_db = has_bias and bool(rng.random() < 0.5)
    kw = dict(
        has_bias=has_bias, compute_dW=compute_dW, compute_db=compute_db,
        reduction=str(rng.choice(["batchmean", "mean", "sum"])),
        temperature=float(rng.choice([0.5, 1.0, 2.0])),
        ignore_frac=float(rng.choice([0.0, 0.0, 0.1, 0.3])),
        w_std=float(rng.choice([0.02, 0.05, 0.1])),
        seed=7000 + i)
    if head in ("kl", "jsd"):
        kw["with_labels"] = bool(rng.random() < 0.7)
    if head in ("selective", "ppo", "cispo"):
        kw["with_weights"] = bool(rng.random() < 0.8)
    if head == "jsd":
        kw.update(H_teacher=8 * int(rng.integers(1, 41)),
                  teacher_has_bias=bool(rng.random() < 0.5),
                  teacher_w_std=float(rng.choice([0.05, 0.1])))
    if head in workloads.RATIO_HEADS:
        low = float(rng.choice([0.1, 0.2]))
        kw.update(clip_low=low, clip_high=float(rng.choice([low, 0.28])),
                  logratio_std=float(rng.choice([0.1, 0.3, 0.5])))
    case = workloads.small_case(BT=BT, H=Hd, V=V, dtype=dtype, head=head, **kw)
    chunk = int(rng.integers(1, BT + 1)) if rng.random() < 0.3 else 0
    logits_bf16 = dtype == "bf16" and bool(rng.random() < 0.25)
    return case, chunk, logits_bf16


N_MEDIUM = 6


def draw_medium(i):
    """Medium case i: bf16, a few thousand tokens and tens of thousands of
    vocabulary entries, so the dX GEMM splits the vocabulary and the batch
    spans several chunks, with the other options drawn as in ``draw``."""
    rng = np.random.default_rng(8000 + i)
    small, chunk, lb = draw(100 + i)
    BT = int(rng.choice([777, 1500, 2100]))
    Hd = 8 * int(rng.integers(32, 129))
    V = int(rng.choice([8191, 16384, 32000, 40000]))
    kw = {}
    if small.head == "jsd":
        kw["H_teacher"] = 8 * int(rng.integers(16, 65))
    case = small.replace(name=f"medium-{small.head}-{BT}x{Hd}x{V}", BT=BT, H=Hd, V=V,
                         dtype="bf16", seed=8000 + i, **kw)
    chunk = int(rng.integers(256, BT + 1)) if rng.random() < 0.3 else 0
    return case, chunk, bool(rng.random() < 0.25)


def test_random_cases_are_valid_plans():
    # host only: every drawn problem is accepted and planned as drawn
    drawn = [draw(i) for i in range(N_CASES)] + [draw_medium(i) for i in range(N_MEDIUM)]
    for i, (case, chunk, lb) in enumerate(drawn):
        prob = fll.make_problem(
            case.BT, case.H, case.V, dtype=case.dtype, head=case.head,
            has_bias=case.has_bias, compute_dW=case.compute_dW,
            compute_db=case.compute_db, reduction=case.reduction,
            ignore_index=case.ignore_index, temperature=case.temperature, eps=case.eps,
            H_teacher=case.H_teacher, teacher_has_bias=case.teacher_has_bias,
            logits_bf16=lb, clip_low=case.clip_low if case.head in workloads.RATIO_HEADS
            else None, clip_high=case.clip_high if case.head in workloads.RATIO_HEADS
            else None)
        plan = fll.fll_plan(prob, 0, chunk)
        if chunk:
            assert plan.chunk_rows == chunk, i
        assert plan.n_chunks * plan.chunk_rows >= case.BT, i


def _parity(case, chunk, lb):
    inp = H.make(case)
    extra = H.fp32_cancellation_floor(inp, case)
    if lb and case.head not in workloads.LABEL_HEADS:
        extra = extra + H.logit_rounding_bound(inp, case)
    out = H.run_gpu(inp, case, chunk_rows=chunk, logits_bf16=lb)
    if chunk:
        assert out["plan"].chunk_rows == chunk
    H.compare_full(out, H.run_oracle(inp, case), case, per_row_atol=extra, inp=inp)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_parity(i):
    case, chunk, lb = draw(i)
    print(f"[random {i}] {case} chunk_rows={chunk} logits_bf16={lb}", flush=True)
    _parity(case, chunk, lb)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_MEDIUM))
def test_random_medium_case_parity(i):
    case, chunk, lb = draw_medium(i)
    print(f"[random medium {i}] {case} chunk_rows={chunk} logits_bf16={lb}", flush=True)
    _parity(case, chunk, lb)


@pytest.mark.parametrize("i", [4, 16, 30])
def test_dlogit_rounding_bound_holds_for_bf16_dlogits(i):
    # host only: the bound the bf16 comparisons admit covers the error that
    # rounding the oracle's dlogits to bf16 alone makes in dX and dW (cases
    # 4 and 16 use sum reduction; there that error exceeds the stated
    # absolute tolerance on a few dW elements, which is what the bound is for)
    import torch

    case, _, _ = draw(i)
    inp = H.make(case)
    ref = H.run_oracle(inp, case)
    dZb = torch.from_numpy(ref["dZ"]).bfloat16().double().numpy()
    bounds = H.dlogit_rounding_bounds(inp, ref, case)
    sims = {"dX": dZb @ H.to_np(inp["W"])}
    if case.compute_dW:
        sims["dW"] = dZb.T @ H.to_np(inp["X"])
    for k, sim in sims.items():
        assert (np.abs(sim - ref[k]) <= bounds[k]).all(), k
