"""The allocation-free entry point, fll_fwd_bwd_static, against fll_fwd_bwd.

Both run the same plan (made for the library's static scratch), so their
outputs must agree bit for bit; two calls in a row, the second on a smaller
problem, show that what the first left in the shared scratch does not leak
into the second. The small problem is also held to the oracle's tolerances.
"""

import pytest
import torch

import workloads
from tests import helpers as H

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(t):
    return None if t is None else t.to(DEV).contiguous()


def _outputs(inp, case):
    X = inp["X"]
    V = inp["W"].shape[0]
    return dict(
        loss=torch.empty((), dtype=torch.float32, device=DEV),
        dX=torch.empty(X.shape, dtype=X.dtype, device=DEV),
        dW=torch.empty(V, X.shape[1], device=DEV) if case.compute_dW else None,
        db=torch.empty(V, device=DEV) if case.compute_db else None,
        per_row=torch.empty(X.shape[0], device=DEV))


def _plan(inp, case):
    import lm_head_projection_token_amd as fll

    prob = fll.make_problem(
        case.BT, case.H, case.V, dtype=case.dtype, head=case.head,
        has_bias=inp["b"] is not None, compute_dW=case.compute_dW,
        compute_db=case.compute_db, reduction=case.reduction,
        ignore_index=case.ignore_index, temperature=case.temperature, eps=case.eps,
        clip_low=case.clip_low if case.head in workloads.RATIO_HEADS else None,
        clip_high=case.clip_high if case.head in workloads.RATIO_HEADS else None)
    return fll.fll_plan(prob, fll.FLL_STATIC_SCRATCH_BYTES)


def _inputs(inp, case):
    kw = dict(X=_dev(inp["X"]), W=_dev(inp["W"]), b=_dev(inp["b"]),
              labels=_dev(inp["labels"]), target=_dev(inp["target"]),
              weights=_dev(inp["weights"]))
    if case.head in workloads.RATIO_HEADS:
        kw["old_logprobs"] = _dev(H.ratio_old_logprobs(inp, case))
    return kw


def _run(inp, case, plan, static):
    import lm_head_projection_token_amd as fll

    kw = _inputs(inp, case)
    out = _outputs(inp, case)
    torch.cuda.synchronize()
    if static:
        before = torch.cuda.memory_allocated()
        fll.fll_fwd_bwd_static(plan, **kw, **out)
        assert torch.cuda.memory_allocated() == before
    else:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
        fll.fll_fwd_bwd(plan, **kw, **out, workspace=ws)
    torch.cuda.synchronize()
    return out


# a head shape near the scratch's limit (several chunks, vocabulary splits),
# then a small ragged problem with a trainable head and bias
BIG = workloads.small_case(BT=2100, H=4096, V=128256, dtype="bf16", head="selective",
                           reduction="mean", ignore_frac=0.05, seed=51)
SMALL = workloads.small_case(BT=300, H=264, V=1000, dtype="bf16", head="kl", has_bias=True,
                             compute_dW=True, compute_db=True, temperature=2.0,
                             ignore_frac=0.1, w_std=0.05, seed=52)


def test_static_entry_point_matches_the_workspace_one_on_two_calls():
    results = []
    for case in (BIG, SMALL):
        print(f"[no-alloc] {case.name}", flush=True)
        inp = H.make(case)
        plan = _plan(inp, case)
        assert plan.n_chunks >= 2
        static = _run(inp, case, plan, static=True)
        ref = _run(inp, case, plan, static=False)
        for k in ("loss", "dX", "dW", "db", "per_row"):
            if ref[k] is not None:
                assert torch.equal(static[k], ref[k]), k
        results.append((inp, case, static))
    inp, case, static = results[-1]
    H.compare_full(static, H.run_oracle(inp, case), case)


def test_static_entry_point_ratio_head_and_repeat():
    case = workloads.small_case(BT=520, H=136, V=777, dtype="bf16", head="ppo",
                                has_bias=True, compute_dW=True, compute_db=True,
                                clip_low=0.2, clip_high=0.28, logratio_std=0.4,
                                ignore_frac=0.05, w_std=0.05, seed=53)
    inp = H.make(case)
    plan = _plan(inp, case)
    a = _run(inp, case, plan, static=True)
    b = _run(inp, case, plan, static=True)
    ref = _run(inp, case, plan, static=False)
    for k in ("loss", "dX", "dW", "db", "per_row"):
        assert torch.equal(a[k], ref[k]) and torch.equal(b[k], ref[k]), k
