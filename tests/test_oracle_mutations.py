"""Planted mistakes in the oracle must fail its pins.

Each mutation below replaces one oracle step (on the CPU, through
monkeypatch) with a plausible slip. The test runs the pin tests of
``test_oracle_pins`` against the mutated oracle and requires that at least
one of them fails. This shows the pins are strong enough to catch the
mistake, not only that the correct oracle passes them.
"""

import numpy as np
import pytest

from oracle import fll_oracle as O
from tests import test_oracle_pins as P

_orig = {name: getattr(O, name) for name in
         ("logits", "kl_rows", "selective_rows", "dlogits", "reduction_scale",
          "valid_rows", "log_softmax", "jsd_rows", "teacher_probs", "ratio_rows",
          "row_weights", "fwd_bwd_blocked")}


def _kl_without_entropy(logP, target, valid, eps):
    L = np.zeros(logP.shape[0])
    r = np.nonzero(valid)[0]
    L[r] = (-np.asarray(target, float)[r] * logP[r]).sum(axis=1)
    return L


def _kl_with_logits_not_logprobs(logP, target, valid, eps):
    # uses S - max instead of S - lse
    return _orig["kl_rows"](logP - logP.max(axis=1, keepdims=True), target, valid, eps)


def _selective_negated(logP, labels, valid):
    return -_orig["selective_rows"](logP, labels, valid)


def _selective_off_by_one(logP, labels, valid):
    y = (np.asarray(labels) + 1) % logP.shape[1]
    y = np.where(np.asarray(labels) == -100, -100, y)
    return _orig["selective_rows"](logP, y, valid)


def _dlogits_no_tau(head, logP, target, labels, w, valid, g, temperature):
    return _orig["dlogits"](head, logP, target, labels, w, valid, g, 1.0)


def _dlogits_q_normalised(head, logP, target, labels, w, valid, g, temperature):
    if head != "kl":
        return _orig["dlogits"](head, logP, target, labels, w, valid, g, temperature)
    dS = np.zeros_like(logP)
    r = np.nonzero(valid)[0]
    q = np.asarray(target, float)[r]
    dS[r] = g * (np.exp(logP[r]) - q)  # assumes sum_v q = 1
    return dS / temperature


def _dlogits_ce_sign_of_selective(head, logP, target, labels, w, valid, g, temperature):
    h = "selective" if head == "ce" else head
    return _orig["dlogits"](h, logP, target, labels, w, valid, g, temperature)


def _dlogits_wrong_sign(head, logP, target, labels, w, valid, g, temperature):
    return -_orig["dlogits"](head, logP, target, labels, w, valid, g, temperature)


def _scale_mean_ignores_V(head, reduction, n_valid, V):
    return _orig["reduction_scale"]("selective", reduction, n_valid, V)


def _scale_counts_ignored(head, reduction, n_valid, V):
    return _orig["reduction_scale"](head, reduction, max(n_valid, 1) + 1, V)


def _logits_drop_bias(X, W, b, temperature):
    return _orig["logits"](X, W, None, temperature)


def _logits_tau_multiplies(X, W, b, temperature):
    return _orig["logits"](X, W, b, 1.0 / temperature)


def _log_softmax_unshifted_lse(S):
    logP, lse = _orig["log_softmax"](S)
    return logP + 1e-3, lse


def _jsd_without_half(logP, teacher, valid):
    return 2.0 * _orig["jsd_rows"](logP, teacher, valid)


def _jsd_as_kl(logP, teacher, valid):
    # KL(teacher || model) in place of the divergence to the mixture
    return _orig["kl_rows"](logP, teacher, valid, 1e-300)


def _dlogits_jsd_no_mean_term(head, logP, target, labels, w, valid, g, temperature):
    if head != "jsd":
        return _orig["dlogits"](head, logP, target, labels, w, valid, g, temperature)
    P = np.exp(logP)
    M = 0.5 * (np.asarray(target) + P)
    with np.errstate(divide="ignore", invalid="ignore"):
        G = np.where(P > 0, 0.5 * np.log(P / M), 0.0)
    dS = g * P * G * valid[:, None]
    return dS / temperature


def _teacher_untempered(X_teacher, W_teacher, b_teacher, temperature):
    return _orig["teacher_probs"](X_teacher, W_teacher, b_teacher, 1.0)


def _valid_all_rows(labels, ignore_index, BT):
    return np.ones(BT, dtype=bool)


def _kl_no_zero_guard(logP, target, valid, eps):
    L = np.zeros(logP.shape[0])
    r = np.nonzero(valid)[0]
    q = np.asarray(target, float)[r]
    with np.errstate(divide="ignore", invalid="ignore"):
        L[r] = (q * np.log(np.maximum(q, eps)) - q * logP[r]).sum(axis=1)
    return L


def _ppo_takes_max(head, logP, labels, valid, old, A, lo, hi):
    L, k = _orig["ratio_rows"](head, logP, labels, valid, old, A, lo, hi)
    if head != "ppo":
        return L, k
    r = np.nonzero(valid)[0]
    lp = logP[r, np.asarray(labels)[r]]
    Ar = np.ones(r.size) if A is None else np.asarray(A, float)[r]
    rho = np.exp(lp - np.asarray(old, float)[r])
    c = np.clip(rho, 1 - lo, 1 + hi)
    L[r] = -np.maximum(rho * Ar, c * Ar)
    k[r] = np.where(rho * Ar >= c * Ar, -rho * Ar, 0.0)
    return L, k


def _ppo_clip_widths_swapped(head, logP, labels, valid, old, A, lo, hi):
    return _orig["ratio_rows"](head, logP, labels, valid, old, A, hi, lo)


def _ppo_grad_through_clip(head, logP, labels, valid, old, A, lo, hi):
    L, k = _orig["ratio_rows"](head, logP, labels, valid, old, A, lo, hi)
    if head == "ppo":
        r = np.nonzero(valid)[0]
        lp = logP[r, np.asarray(labels)[r]]
        Ar = np.ones(r.size) if A is None else np.asarray(A, float)[r]
        k[r] = -np.exp(lp - np.asarray(old, float)[r]) * Ar
    return L, k


def _ratio_inverted(head, logP, labels, valid, old, A, lo, hi):
    # rho = exp(old - new): the old log-probs reflected about the new ones
    r = np.nonzero(valid)[0]
    lp = np.zeros(logP.shape[0])
    lp[r] = logP[r, np.asarray(labels)[r]]
    return _orig["ratio_rows"](head, logP, labels, valid, 2 * lp - np.asarray(old, float),
                               A, lo, hi)


def _cispo_grad_through_weight(head, logP, labels, valid, old, A, lo, hi):
    L, k = _orig["ratio_rows"](head, logP, labels, valid, old, A, lo, hi)
    if head == "cispo":
        r = np.nonzero(valid)[0]
        lp = logP[r, np.asarray(labels)[r]]
        Ar = np.ones(r.size) if A is None else np.asarray(A, float)[r]
        rho = np.exp(lp - np.asarray(old, float)[r])
        inside = (rho > 1 - lo) & (rho < 1 + hi)
        k[r] = k[r] - Ar * lp * rho * inside
    return L, k


def _ratio_weighted_twice(head, weights, BT):
    if head in ("ppo", "cispo") and weights is not None:
        return np.asarray(weights, float)
    return _orig["row_weights"](head, weights, BT)


def _blocked_drops_last_block(X, W, b=None, **kw):
    out = _orig["fwd_bwd_blocked"](X, W, b, **kw)
    blk = kw.get("block_rows", 512)
    last = ((X.shape[0] - 1) // blk) * blk
    if last > 0:
        out["dX"][last:] = 0.0
    return out


MUTATIONS = {
    "kl drops sum q log q": ("kl_rows", _kl_without_entropy),
    "kl uses S - max": ("kl_rows", _kl_with_logits_not_logprobs),
    "selective negated": ("selective_rows", _selective_negated),
    "selective label off by one": ("selective_rows", _selective_off_by_one),
    "dZ misses 1/tau": ("dlogits", _dlogits_no_tau),
    "KL grad assumes sum q = 1": ("dlogits", _dlogits_q_normalised),
    "gradient sign flipped": ("dlogits", _dlogits_wrong_sign),
    "CE gradient takes the selective sign": ("dlogits", _dlogits_ce_sign_of_selective),
    "KL mean ignores V": ("reduction_scale", _scale_mean_ignores_V),
    "ignored rows counted": ("reduction_scale", _scale_counts_ignored),
    "bias dropped": ("logits", _logits_drop_bias),
    "tau multiplies": ("logits", _logits_tau_multiplies),
    "log-softmax off by a constant": ("log_softmax", _log_softmax_unshifted_lse),
    "ignore mask ignored": ("valid_rows", _valid_all_rows),
    "JSD drops the one-half": ("jsd_rows", _jsd_without_half),
    "JSD replaced by KL to the teacher": ("jsd_rows", _jsd_as_kl),
    "JSD gradient misses the mean term": ("dlogits", _dlogits_jsd_no_mean_term),
    "teacher logits not tempered": ("teacher_probs", _teacher_untempered),
    "KL zero entries not guarded": ("kl_rows", _kl_no_zero_guard),
    "PPO takes the max": ("ratio_rows", _ppo_takes_max),
    "PPO clip widths swapped": ("ratio_rows", _ppo_clip_widths_swapped),
    "PPO gradient through the clipped product": ("ratio_rows", _ppo_grad_through_clip),
    "ratio inverted": ("ratio_rows", _ratio_inverted),
    "CISPO gradient through its weight": ("ratio_rows", _cispo_grad_through_weight),
    "ratio heads weighted twice": ("row_weights", _ratio_weighted_twice),
    "blocked pass drops its last block": ("fwd_bwd_blocked", _blocked_drops_last_block),
}


def _pin_tests():
    tests = []
    for name in dir(P):
        if not name.startswith("test_"):
            continue
        fn = getattr(P, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            tests.append((name, fn, {}))
            continue
        # stacked parametrize marks: every combination
        combos = [{}]
        for m in params:
            names = [a.strip() for a in m.args[0].split(",")]
            combos = [dict(c, **dict(zip(names, v if isinstance(v, tuple) else (v,))))
                      for c in combos for v in m.args[1]]
        for kw in combos:
            if name == "test_gradients_central_differences" and kw["tau"] != 2.0:
                continue  # one temperature suffices here; keeps the run short
            tests.append((f"{name}{tuple(kw.values())}", fn, kw))
    return tests


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_mutation(mutation, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for name, test, kwargs in _pin_tests():
        try:
            test(**kwargs)
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    assert caught, f"no pin fails when the oracle has the slip: {mutation}"
