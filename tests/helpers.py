"""Shared helpers of the tests: run the HIP path, run the oracle, compare.

Tolerances (stated for the method's float configurations):
  fp32 problems: loss and every gradient within rtol 1e-5, with an absolute
    floor of 1e-5 * max|reference| per tensor.
  bf16 problems: loss relative error <= 2e-3; gradients within atol 1e-2 /
    rtol 2e-2 as stated; because 1/n scaling makes gradient entries tiny
    (~1e-5), that literal check is vacuous, so gradients must also pass the
    same rtol with atol = 1e-2 * max|reference| and a relative Frobenius
    error <= 1e-2.
"""

from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import workloads

RATIO_MARGIN = 1e-3  # log-ratios kept this far from the clip edges (see below)


def to_np(t):
    return None if t is None else t.detach().cpu().double().numpy()


def ratio_old_logprobs(inp, case, margin=RATIO_MARGIN, block_rows=512):
    """The ratio heads' old log-probs: old_r = log p(y_r) - d_r, with log p(y_r)
    from the oracle and d_r the drawn log-ratio, as float32 (the GPU's input;
    the oracle then reads the same values). A drawn d_r within ``margin`` of a
    clip edge (log(1 + clip_high), log(1 - clip_low)) is moved 2 * margin
    away from it: there the clip decision turns on the last bits of log p(y),
    which float32 logits on the GPU and float64 ones in the oracle need not
    share, and either branch would be right. Cached in ``inp``."""
    if inp.get("old_logprobs") is not None:
        return inp["old_logprobs"]
    from oracle import fll_oracle

    d = inp["logratio"].double().numpy().copy()
    edges = [math.log1p(case.clip_high)]
    if case.clip_low < 1.0:
        edges.append(math.log1p(-case.clip_low))
    for e in edges:
        near = np.abs(d - e) < margin
        d[near] = e + np.where(d[near] >= e, 2 * margin, -2 * margin)
    labels = inp["labels"].numpy()
    lp = fll_oracle.label_logprobs(
        to_np32(inp["X"]), to_np32(inp["W"]), to_np(inp["b"]), labels,
        temperature=case.temperature, ignore_index=case.ignore_index,
        block_rows=block_rows)
    old = torch.from_numpy((lp - d).astype(np.float32))
    old[inp["labels"] == case.ignore_index] = float("nan")  # never read
    inp["old_logprobs"] = old
    return old


def to_np32(t):
    """float32 numpy view of a CPU tensor (bf16 and fp32 values are exact)."""
    return None if t is None else t.detach().cpu().float().numpy()


def run_gpu(inp, case, chunk_rows=0, per_row=True, device="cuda:0", logits_bf16=False):
    import lm_head_projection_token_amd as fll

    def dev(t):
        return None if t is None else t.to(device).contiguous()

    ratio = {}
    if case.head in workloads.RATIO_HEADS:
        ratio = dict(old_logprobs=dev(ratio_old_logprobs(inp, case)),
                     clip_low=case.clip_low, clip_high=case.clip_high)

    out = fll.fused_lm_head_loss(
        dev(inp["X"]), dev(inp["W"]), dev(inp["b"]), head=case.head,
        labels=dev(inp["labels"]), target=dev(inp["target"]), weights=dev(inp["weights"]),
        reduction=case.reduction, ignore_index=case.ignore_index,
        temperature=case.temperature, eps=case.eps, compute_dW=case.compute_dW,
        compute_db=case.compute_db, chunk_rows=chunk_rows, per_row=per_row,
        X_teacher=dev(inp.get("X_teacher")), W_teacher=dev(inp.get("W_teacher")),
        b_teacher=dev(inp.get("b_teacher")), logits_bf16=logits_bf16, **ratio)
    torch.cuda.synchronize()
    return out


def _ratio_kw(inp, case):
    if case.head not in workloads.RATIO_HEADS:
        return {}
    return dict(old_logprobs=to_np(ratio_old_logprobs(inp, case)),
                clip_low=case.clip_low, clip_high=case.clip_high)


def run_oracle_blocked(inp, case, block_rows=512, tag=""):
    """The oracle's row-blocked pass over the whole batch (the same arithmetic
    as ``fwd_bwd``), printing its progress every ~20 % of the rows."""
    from oracle import fll_oracle

    t0 = time.time()
    marks = set()

    def progress(done, total):
        pct = int(100 * done / total) // 20 * 20
        if pct not in marks:
            marks.add(pct)
            print(f"[oracle {tag}] {done}/{total} rows, {time.time() - t0:.0f} s",
                  flush=True, file=sys.stderr)

    return fll_oracle.fwd_bwd_blocked(
        to_np32(inp["X"]), to_np32(inp["W"]), to_np(inp["b"]), head=case.head,
        labels=None if inp["labels"] is None else inp["labels"].numpy(),
        target=None if inp["target"] is None else inp["target"].numpy(),
        weights=to_np(inp["weights"]), reduction=case.reduction,
        ignore_index=case.ignore_index, temperature=case.temperature, eps=case.eps,
        compute_dW=case.compute_dW, compute_db=case.compute_db,
        X_teacher=to_np32(inp.get("X_teacher")), W_teacher=to_np32(inp.get("W_teacher")),
        b_teacher=to_np(inp.get("b_teacher")), block_rows=block_rows, progress=progress,
        **_ratio_kw(inp, case))


def run_oracle(inp, case):
    from oracle import fll_oracle

    return fll_oracle.fwd_bwd(
        to_np(inp["X"]), to_np(inp["W"]), to_np(inp["b"]), head=case.head,
        labels=None if inp["labels"] is None else inp["labels"].numpy(),
        target=to_np(inp["target"]), weights=to_np(inp["weights"]),
        reduction=case.reduction, ignore_index=case.ignore_index,
        temperature=case.temperature, eps=case.eps, compute_dW=case.compute_dW,
        compute_db=case.compute_db, X_teacher=to_np(inp.get("X_teacher")),
        W_teacher=to_np(inp.get("W_teacher")), b_teacher=to_np(inp.get("b_teacher")),
        **_ratio_kw(inp, case))


def check_loss(gpu_loss: float, ref: float, dtype: str, what="loss"):
    tol = 1e-5 if dtype == "fp32" else 2e-3
    err = abs(gpu_loss - ref)
    assert err <= tol * max(abs(ref), 1e-30) or err <= 1e-30, \
        f"{what}: gpu {gpu_loss!r} vs oracle {ref!r} (rel {err / max(abs(ref), 1e-300):.3e})"


def _row_blocks(n, elems_per_row, target=1 << 24):
    step = max(1, target // max(1, elems_per_row))
    return [slice(i, min(n, i + step)) for i in range(0, max(n, 1), step)]


def check_grad(got, ref, dtype: str, what: str, bound=None):
    """Element-wise gradient check at the stated tolerances (see the module
    docstring). Large arrays (a full V x H weight gradient) are compared in
    row blocks with the same per-tensor scale and Frobenius norms, so no
    temporary of the whole array's size is formed. ``bound`` (bf16, same
    shape): an element outside the stated tolerance still passes that check
    when its error is within bound, the rounding bound of the bf16 dlogits
    (see ``dlogit_rounding_bounds``); the scaled and Frobenius checks apply
    to every element regardless."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, what
    if ref.size == 0:
        return
    n = ref.shape[0]
    per_row = int(ref.size // max(n, 1))
    blocks = _row_blocks(n, per_row)
    scale = max(float(np.abs(ref[blk]).max()) for blk in blocks)
    num = den = 0.0
    for blk in blocks:
        g = np.asarray(got[blk], dtype=np.float64)
        r = np.asarray(ref[blk], dtype=np.float64)
        assert np.isfinite(g).all(), f"{what}: non-finite values"
        if dtype == "fp32":
            np.testing.assert_allclose(g, r, rtol=1e-5, atol=1e-5 * scale, err_msg=what)
            continue
        if bound is None:
            np.testing.assert_allclose(g, r, rtol=2e-2, atol=1e-2, err_msg=what + " (stated)")
        else:
            err = np.abs(g - r)
            bad = err > np.maximum(1e-2 + 2e-2 * np.abs(r), np.asarray(bound[blk]))
            assert not bad.any(), \
                (f"{what} (stated, or within the dlogit rounding bound): {int(bad.sum())} "
                 f"elements out, max error {float(err[bad].max()):.3e}")
        np.testing.assert_allclose(g, r, rtol=2e-2, atol=1e-2 * scale,
                                   err_msg=what + " (scaled)")
        num += float(np.square(g - r).sum())
        den += float(np.square(r).sum())
    if dtype == "fp32":
        return
    if den > 0:
        rel = math.sqrt(num / den)
        assert rel <= 1e-2, f"{what}: relative Frobenius error {rel:.3e}"
    else:
        assert num == 0.0, f"{what}: expected exact zeros"


BF16_UNIT_ROUNDOFF = 2.0 ** -8


def logit_rounding_bound(inp, case, rows=None):
    """Per-row bound on how far rounding the chunk logits to bf16 can move a
    per-row loss term, to first order: every logit moves by at most
    u |S_rv| (u = 2^-8), and each head's term has a logit gradient whose
    absolute row sum is at most 2 (the label's logit and the log-sum-exp; the
    target's logits and the log-sum-exp; for JSD the same for each side), so
    |d L_r| <= 2 u (max_v |S_rv| + max_v |T_rv|) with T the teacher's logits."""
    def row_max(X, W, b):
        X = X.double() if rows is None else X[rows].double()
        S = X @ W.double().T
        if b is not None:
            S = S + b.double()
        return (S / case.temperature).abs().max(dim=1).values.numpy()

    m = row_max(inp["X"], inp["W"], inp["b"])
    if inp.get("X_teacher") is not None:
        m = m + row_max(inp["X_teacher"], inp["W_teacher"], inp.get("b_teacher"))
    return 2.0 * BF16_UNIT_ROUNDOFF * m


def dlogit_rounding_bounds(inp, ref, case):
    """bf16 problems: how far each gradient element may move because the
    method rounds the dlogits dZ to bf16 before the dX / dW GEMMs (round to
    nearest, relative error <= u = 2^-8) and sums K products in float32
    (first order: K 2^-24 of the sum of magnitudes): for a gradient
    sum_k a_k b_k, |error| <= (u + K 2^-24) sum_k |a_k b_k|. With sum
    reduction the gradients are of order one and an element that is a
    cancellation of larger terms can exceed the stated absolute tolerance
    by this rounding alone. Uses the oracle's dZ."""
    dZ = np.abs(ref["dZ"])
    BT, V = dZ.shape
    eps32 = 2.0 ** -24
    out = {"dX": (BF16_UNIT_ROUNDOFF + V * eps32) * (dZ @ np.abs(to_np(inp["W"])))}
    if case.compute_dW:
        out["dW"] = (BF16_UNIT_ROUNDOFF + BT * eps32) * (dZ.T @ np.abs(to_np(inp["X"])))
    if case.compute_db:
        out["db"] = (BF16_UNIT_ROUNDOFF + BT * eps32) * dZ.sum(axis=0)
    return out


def fp32_cancellation_floor(inp, case):
    """Per-row absolute floor for per-row terms whose reference is (near)
    zero: the kernels form them in float32 as differences of terms as large
    as the row's largest logit (KL: sum q S against the log-sum-exp; label
    heads: S_y against it), so a few float32 ulps of max_v |S_rv| (and of
    the teacher's logits) remain where the exact value is 0 (a one-entry
    vocabulary)."""
    def row_max(X, W, b):
        S = X.double() @ W.double().T
        if b is not None:
            S = S + b.double()
        return (S / case.temperature).abs().max(dim=1).values.numpy()

    m = row_max(inp["X"], inp["W"], inp["b"])
    if inp.get("X_teacher") is not None:
        m = m + row_max(inp["X_teacher"], inp["W_teacher"], inp.get("b_teacher"))
    return 8.0 * 2.0 ** -24 * (1.0 + m)


def compare_full(out, ref, case, per_row_atol=None, inp=None):
    """Loss and gradients at the stated tolerances; per-row terms at the
    loss tolerance, plus per_row_atol (a per-row array) when given. With
    ``inp`` (bf16 problems, oracle results from ``fwd_bwd``), the stated
    gradient check also admits errors within ``dlogit_rounding_bounds``."""
    check_loss(float(out["loss"]), ref["loss"], case.dtype)
    if out.get("per_row") is not None:
        per = to_np(out["per_row"])
        tol = 1e-5 if case.dtype == "fp32" else 2e-3
        scale = float(np.abs(ref["per_row"]).max()) if ref["per_row"].size else 0.0
        atol = tol * scale if per_row_atol is None else tol * scale + per_row_atol
        err = np.abs(per - ref["per_row"])
        bad = err > atol + tol * np.abs(ref["per_row"])
        assert not bad.any(), \
            f"per_row: {int(bad.sum())} rows out of tolerance, max err {err.max():.3e}"
    bounds = {}
    if inp is not None and case.dtype == "bf16" and ref.get("dZ") is not None:
        bounds = dlogit_rounding_bounds(inp, ref, case)
    check_grad(to_np(out["dX"]), ref["dX"], case.dtype, "dX", bounds.get("dX"))
    if case.compute_dW:
        check_grad(to_np(out["dW"]), ref["dW"], case.dtype, "dW", bounds.get("dW"))
    if case.compute_db:
        check_grad(to_np(out["db"]), ref["db"], case.dtype, "db", bounds.get("db"))


def make(case):
    return workloads.make_inputs(case)
