"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the pages and the mathematics fix:
closed forms, invariants (Gibbs' inequality, zero row sums of the
log-softmax backward), special cases that reduce to torch library routines
evaluated in float64 (``log_softmax``, ``cross_entropy``, ``kl_div``,
autograd), central finite differences and an exact temperature identity.
They are chosen so that a plausible slip in the oracle -- a dropped term, a
wrong sign, a wrong index, a transposed operand, a missing 1/tau, a wrong
denominator -- fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import fll_oracle as O

rng = np.random.default_rng(20261202)


def _rand(*shape, std=1.0):
    return rng.normal(0.0, std, size=shape)


def _softmax(a):
    e = np.exp(a - a.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# logits and log-softmax
# --------------------------------------------------------------------------

def test_logits_match_torch_linear():
    X, W, b = _rand(7, 5), _rand(11, 5), _rand(11)
    S = O.logits(X, W, b, 2.0)
    ref = F.linear(torch.tensor(X), torch.tensor(W), torch.tensor(b)) / 2.0
    np.testing.assert_allclose(S, ref.numpy(), rtol=1e-14, atol=1e-14)
    assert S.shape == (7, 11)


def test_log_softmax_closed_form_uniform():
    # W = 0, b = 0: every logit is 0, so log p = -log V exactly.
    for V in (1, 2, 7, 1000):
        S = O.logits(_rand(3, 4), np.zeros((V, 4)), np.zeros(V), 1.0)
        logP, lse = O.log_softmax(S)
        np.testing.assert_allclose(logP, -math.log(V), rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, math.log(V), rtol=0, atol=1e-15)


def test_log_softmax_two_class_closed_form():
    # logits [0, log 3] -> p = [1/4, 3/4].
    S = np.array([[0.0, math.log(3.0)]])
    logP, _ = O.log_softmax(S)
    np.testing.assert_allclose(logP[0], [math.log(0.25), math.log(0.75)], rtol=1e-15)


def test_log_softmax_matches_torch_and_shift_invariance():
    S = _rand(6, 50, std=5.0)
    logP, _ = O.log_softmax(S)
    np.testing.assert_allclose(logP, torch.log_softmax(torch.tensor(S), 1).numpy(),
                               rtol=1e-13, atol=1e-13)
    shifted, _ = O.log_softmax(S + _rand(6, 1, std=100.0))
    np.testing.assert_allclose(shifted, logP, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.exp(logP).sum(1), 1.0, rtol=1e-14)


# --------------------------------------------------------------------------
# KL head
# --------------------------------------------------------------------------

def _kl_case(BT=9, H=6, V=13, tau=1.0, bias=True):
    X, W = _rand(BT, H), _rand(V, H)
    b = _rand(V) if bias else None
    q = _softmax(_rand(BT, V, std=2.0))
    return X, W, b, q


def test_kl_two_class_closed_form():
    # p = [1/4, 3/4], q = [1/2, 1/2]: KL = 1/2 log 2 + 1/2 log(2/3) = 1/2 log(4/3),
    # dS = Q p - q = [-1/4, 1/4].
    X = np.array([[1.0]])
    W = np.array([[0.0], [math.log(3.0)]])
    q = np.array([[0.5, 0.5]])
    out = O.fwd_bwd(X, W, head="kl", target=q, reduction="sum")
    assert out["loss"] == pytest.approx(0.5 * math.log(4.0 / 3.0), rel=1e-15)
    # dX = dZ W = -1/4 * 0 + 1/4 * log 3
    assert out["dX"][0, 0] == pytest.approx(0.25 * math.log(3.0), rel=1e-15)
    np.testing.assert_allclose(out["db"], [-0.25, 0.25], rtol=1e-15)
    np.testing.assert_allclose(out["dW"][:, 0], [-0.25, 0.25], rtol=1e-15)


def test_kl_zero_when_target_is_model_softmax():
    # eps = 0: the clamp would replace q log q by q log eps for q < eps and
    # move the loss off 0 by up to eps |log eps| per such entry; without it
    # the invariant holds to rounding. Own generator: the draws do not
    # depend on which tests ran before.
    g = np.random.default_rng(7)
    X, W, b = g.normal(size=(9, 6)), g.normal(size=(13, 6)), g.normal(size=13)
    for tau in (0.5, 1.0, 2.0):
        S = O.logits(X, W, b, tau)
        q = _softmax(S)
        out = O.fwd_bwd(X, W, b, head="kl", target=q, temperature=tau,
                        reduction="sum", eps=0.0)
        # KL = sum q log q - sum q log p cancels two sums of size ~|S|; fp64
        # rounding leaves a few ulps of their magnitude
        scale = float(np.abs(q * np.log(q)).sum() + np.abs(q * S).sum())
        assert abs(out["loss"]) < 1e-14 * max(scale, 1.0) * 100
        assert np.abs(out["dX"]).max() < 1e-13
        assert np.abs(out["dW"]).max() < 1e-13
        assert np.abs(out["db"]).max() < 1e-13


def test_kl_nonnegative():
    for seed in range(5):
        X, W, b, q = _kl_case()
        out = O.fwd_bwd(X, W, b, head="kl", target=q, reduction="sum")
        assert (out["per_row"] >= -1e-14).all()
        assert out["loss"] > 0


@pytest.mark.parametrize("reduction", ["batchmean", "sum", "mean"])
def test_kl_matches_torch_kl_div(reduction):
    X, W, b, q = _kl_case(BT=12, V=17)
    q[0, 3] = 0.0  # an exact zero: 0 * log 0 must contribute 0
    q[0] /= q[0].sum()
    for tau in (0.5, 2.0):
        out = O.fwd_bwd(X, W, b, head="kl", target=q, temperature=tau,
                        reduction=reduction)
        logP = torch.log_softmax(torch.tensor(O.logits(X, W, b, tau)), 1)
        ref = F.kl_div(logP, torch.tensor(q), reduction=reduction, log_target=False)
        assert out["loss"] == pytest.approx(float(ref), rel=1e-12)


def test_kl_ignored_rows_leave_the_batch():
    X, W, b, q = _kl_case(BT=10, V=9)
    labels = np.arange(10)
    labels[[1, 4, 7]] = -100
    q_nan = q.copy()
    q_nan[[1, 4, 7]] = np.nan  # never read
    out = O.fwd_bwd(X, W, b, head="kl", target=q_nan, labels=labels,
                    reduction="batchmean")
    keep = labels != -100
    logP = torch.log_softmax(torch.tensor(O.logits(X[keep], W, b, 1.0)), 1)
    ref = F.kl_div(logP, torch.tensor(q[keep]), reduction="batchmean")
    assert out["n_valid"] == 7
    assert out["loss"] == pytest.approx(float(ref), rel=1e-12)
    assert np.isfinite(out["dX"]).all()
    assert (out["dX"][~keep] == 0).all()
    # moving ignored rows' inputs changes nothing
    X2 = X.copy()
    X2[~keep] += 10.0
    out2 = O.fwd_bwd(X2, W, b, head="kl", target=q_nan, labels=labels)
    assert out2["loss"] == out["loss"]
    np.testing.assert_array_equal(out2["dX"][keep], out["dX"][keep])


def test_kl_one_hot_target_is_cross_entropy():
    X, W, b, _ = _kl_case(BT=8, V=11)
    y = rng.integers(0, 11, size=8)
    q = np.zeros((8, 11))
    q[np.arange(8), y] = 1.0
    out = O.fwd_bwd(X, W, b, head="kl", target=q, reduction="sum")
    ce = F.cross_entropy(torch.tensor(O.logits(X, W, b, 1.0)), torch.tensor(y),
                         reduction="none")
    np.testing.assert_allclose(out["per_row"], ce.numpy(), rtol=1e-13)


def test_kl_reduction_identities():
    X, W, b, q = _kl_case(BT=6, V=10)
    labels = np.array([0, -100, 2, 3, -100, 5])
    o = {r: O.fwd_bwd(X, W, b, head="kl", target=q, labels=labels, reduction=r)
         for r in ("batchmean", "mean", "sum")}
    n, V = 4, 10
    assert o["sum"]["loss"] == pytest.approx(n * o["batchmean"]["loss"], rel=1e-14)
    assert o["sum"]["loss"] == pytest.approx(n * V * o["mean"]["loss"], rel=1e-14)
    np.testing.assert_allclose(o["sum"]["dX"], n * o["batchmean"]["dX"], rtol=1e-13)


def test_reduction_none_refused():
    with pytest.raises(ValueError):
        O.reduction_scale("kl", "none", 3, 5)


def test_no_valid_rows_gives_zero():
    X, W, b, q = _kl_case(BT=4, V=5)
    labels = np.full(4, -100)
    out = O.fwd_bwd(X, W, b, head="kl", target=np.full((4, 5), np.nan),
                    labels=labels)
    assert out["loss"] == 0.0 and out["n_valid"] == 0
    assert (out["dX"] == 0).all() and (out["dW"] == 0).all() and (out["db"] == 0).all()


# --------------------------------------------------------------------------
# selective head
# --------------------------------------------------------------------------

def test_selective_matches_negative_cross_entropy():
    X, W, b = _rand(10, 6), _rand(15, 6), _rand(15)
    y = rng.integers(0, 15, size=10)
    y[3] = -100
    out = O.fwd_bwd(X, W, b, head="selective", labels=y, reduction="mean")
    ce = F.cross_entropy(torch.tensor(O.logits(X, W, b, 1.0)), torch.tensor(y),
                         ignore_index=-100, reduction="mean")
    assert out["loss"] == pytest.approx(-float(ce), rel=1e-13)


def test_selective_weighted_matches_torch():
    X, W = _rand(10, 6), _rand(15, 6)
    y = rng.integers(0, 15, size=10)
    w = _rand(10)
    for tau in (0.5, 1.0):
        out = O.fwd_bwd(X, W, head="selective", labels=y, weights=w,
                        temperature=tau, reduction="mean")
        ce = F.cross_entropy(torch.tensor(O.logits(X, W, None, tau)),
                             torch.tensor(y), reduction="none")
        ref = -(torch.tensor(w) * ce).sum() / 10
        assert out["loss"] == pytest.approx(float(ref), rel=1e-13)
        assert (out["per_row"] <= 0).all()


def test_selective_uniform_logits_closed_form():
    V = 37
    X = _rand(8, 4)
    y = rng.integers(0, V, size=8)
    w = _rand(8)
    out = O.fwd_bwd(X, np.zeros((V, 4)), np.zeros(V), head="selective",
                    labels=y, weights=w, reduction="mean")
    assert out["loss"] == pytest.approx(-math.log(V) * w.sum() / 8, rel=1e-14)


def test_selective_label_out_of_range_raises():
    with pytest.raises(ValueError):
        O.fwd_bwd(_rand(2, 3), _rand(4, 3), head="selective", labels=np.array([0, 4]))


# --------------------------------------------------------------------------
# gradients
# --------------------------------------------------------------------------

def _loss_fn(kw):
    def f(X, W, b):
        return O.fwd_bwd(X, W, b, **kw)["loss"]
    return f


def _central_fd(f, args, i, h=1e-6):
    base = [a.copy() if a is not None else None for a in args]
    g = np.zeros_like(base[i])
    it = np.nditer(base[i], flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        p = [a.copy() if a is not None else None for a in base]
        m = [a.copy() if a is not None else None for a in base]
        p[i][idx] += h
        m[i][idx] -= h
        g[idx] = (f(*p) - f(*m)) / (2 * h)
    return g


FD_CASES = []
for head in ("kl", "selective", "ce", "jsd"):
    for reduction in ("batchmean", "mean", "sum"):
        for tau in (0.5, 1.0, 2.0):
            FD_CASES.append((head, reduction, tau))


@pytest.mark.parametrize("head,reduction,tau", FD_CASES)
def test_gradients_central_differences(head, reduction, tau):
    BT, H, V = 5, 4, 7
    X, W, b = _rand(BT, H), _rand(V, H), _rand(V)
    labels = rng.integers(0, V, size=BT)
    labels[2] = -100
    kw = dict(head=head, labels=labels, reduction=reduction, temperature=tau)
    if head == "kl":
        q = _softmax(_rand(BT, V)) * 1.3  # unnormalised: exercises Q_r
        kw["target"] = q
    elif head == "jsd":
        kw.update(X_teacher=_rand(BT, 6), W_teacher=_rand(V, 6), b_teacher=_rand(V))
    else:
        kw["weights"] = _rand(BT)
    out = O.fwd_bwd(X, W, b, **kw)
    f = _loss_fn(kw)
    for i, name in ((0, "dX"), (1, "dW"), (2, "db")):
        fd = _central_fd(f, [X, W, b], i)
        np.testing.assert_allclose(out[name], fd, rtol=1e-6, atol=1e-8,
                                   err_msg=name)


@pytest.mark.parametrize("head", ["kl", "selective", "ce", "jsd"])
def test_gradients_match_torch_autograd(head):
    BT, H, V, tau = 33, 24, 57, 2.0
    X, W, b = _rand(BT, H), _rand(V, H, std=0.3), _rand(V)
    labels = rng.integers(0, V, size=BT)
    labels[::7] = -100
    keep = labels != -100
    Xt, Wt, bt = (torch.tensor(a, requires_grad=True) for a in (X, W, b))
    logP = torch.log_softmax(F.linear(Xt, Wt, bt) / tau, dim=1)
    if head == "kl":
        q = _softmax(_rand(BT, V, std=2.0))
        loss_t = F.kl_div(logP[torch.tensor(keep)], torch.tensor(q[keep]),
                          reduction="batchmean")
        kw = dict(target=q, reduction="batchmean")
    elif head == "selective":
        w = _rand(BT)
        ce = F.cross_entropy(F.linear(Xt, Wt, bt) / tau, torch.tensor(labels),
                             ignore_index=-100, reduction="none")
        loss_t = -(torch.tensor(w) * ce).sum() / keep.sum()
        kw = dict(weights=w, reduction="mean")
    elif head == "ce":
        loss_t = F.cross_entropy(F.linear(Xt, Wt, bt) / tau, torch.tensor(labels),
                                 ignore_index=-100, reduction="mean")
        kw = dict(reduction="mean")
    else:
        # the Jensen-Shannon divergence written out in torch, differentiated
        # through the mixture M by autograd (teacher: no gradient)
        Xte, Wte, bte = _rand(BT, 40), _rand(V, 40, std=0.3), _rand(V)
        logPt = torch.log_softmax(F.linear(*(torch.tensor(a) for a in (Xte, Wte, bte))) / tau, 1)
        Pt, Q = logPt.exp(), logP.exp()
        logM = torch.log(0.5 * (Pt + Q))
        js = 0.5 * (Pt * (logPt - logM)).sum(1) + 0.5 * (Q * (logP - logM)).sum(1)
        loss_t = js[torch.tensor(keep)].sum() / keep.sum()
        kw = dict(reduction="batchmean", X_teacher=Xte, W_teacher=Wte, b_teacher=bte)
    loss_t.backward()
    out = O.fwd_bwd(X, W, b, head=head, labels=labels, temperature=tau, **kw)
    assert out["loss"] == pytest.approx(float(loss_t), rel=1e-12)
    np.testing.assert_allclose(out["dX"], Xt.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["db"], bt.grad.numpy(), rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("head", ["kl", "selective", "jsd"])
def test_dlogit_rows_sum_to_zero(head):
    BT, V = 20, 300
    logP, _ = O.log_softmax(_rand(BT, V, std=3.0))
    labels = rng.integers(0, V, size=BT)
    q = _softmax(_rand(BT, V)) * 0.7  # sum_v (Q p - q) = 0 for any scale
    if head == "jsd":
        q = _softmax(_rand(BT, V, std=3.0))  # the teacher distribution
    dZ = O.dlogits(head, logP, q, labels, _rand(BT), np.ones(BT, bool), 0.3, 2.0)
    np.testing.assert_allclose(dZ.sum(axis=1), 0.0, atol=1e-15)


@pytest.mark.parametrize("head", ["kl", "selective", "jsd"])
def test_temperature_power_of_two_identity(head):
    # S = (X W^T + b)/tau equals X (W/tau)^T + b/tau exactly for tau = 2^k, so
    # dX must agree bitwise, and dW(tau) = dW'(tau=1) / tau: pins where 1/tau
    # enters the forward and the backward.
    BT, H, V = 9, 8, 21
    X, W, b = _rand(BT, H), _rand(V, H), _rand(V)
    labels = rng.integers(0, V, size=BT)
    kw = dict(head=head, labels=labels)
    Xte, Wte, bte = _rand(BT, 6), _rand(V, 6), _rand(V)
    if head == "kl":
        kw["target"] = _softmax(_rand(BT, V))
    elif head != "jsd":
        kw["weights"] = _rand(BT)
    for tau in (0.5, 2.0, 4.0):
        if head == "jsd":  # the temperature divides the teacher's logits too
            kw.update(X_teacher=Xte, W_teacher=Wte, b_teacher=bte)
            a = O.fwd_bwd(X, W, b, temperature=tau, **kw)
            kw.update(W_teacher=Wte / tau, b_teacher=bte / tau)
            c = O.fwd_bwd(X, W / tau, b / tau, temperature=1.0, **kw)
        else:
            a = O.fwd_bwd(X, W, b, temperature=tau, **kw)
            c = O.fwd_bwd(X, W / tau, b / tau, temperature=1.0, **kw)
        assert a["loss"] == c["loss"]
        np.testing.assert_array_equal(a["dX"], c["dX"])
        np.testing.assert_array_equal(a["dW"], c["dW"] / tau)
        np.testing.assert_array_equal(a["db"], c["db"] / tau)


def test_flags_do_not_change_dx():
    X, W, b, q = _kl_case()
    a = O.fwd_bwd(X, W, b, head="kl", target=q, compute_dW=False, compute_db=False)
    c = O.fwd_bwd(X, W, b, head="kl", target=q, compute_dW=True, compute_db=True)
    assert a["dW"] is None and a["db"] is None
    np.testing.assert_array_equal(a["dX"], c["dX"])
    assert a["loss"] == c["loss"]


@pytest.mark.parametrize("head", ["kl", "selective", "ce", "jsd", "ppo", "cispo"])
def test_sampled_rows_agree_with_full(head):
    BT, H, V = 16, 8, 29
    X, W, b = _rand(BT, H), _rand(V, H), _rand(V)
    labels = rng.integers(0, V, size=BT)
    labels[[3, 9]] = -100
    kw = dict(head=head, reduction="mean", temperature=2.0)
    q = w = None
    tk = tsub = {}
    if head == "kl":
        q = _softmax(_rand(BT, V))
    elif head == "jsd":
        Xte, Wte, bte = _rand(BT, 5), _rand(V, 5), _rand(V)
        tk = dict(X_teacher=Xte, W_teacher=Wte, b_teacher=bte)
    else:
        w = _rand(BT)
    if head in ("ppo", "cispo"):
        old = _torch_logp_label(X, W, b, labels, 2.0) - _rand(BT, std=0.3)
        tk = dict(old_logprobs=old, clip_low=0.2, clip_high=0.28)
    full = O.fwd_bwd(X, W, b, labels=labels, target=q, weights=w, **kw, **tk)
    rows = np.array([0, 3, 5, 15])
    if head == "jsd":
        tsub = dict(Xt_rows=Xte[rows], W_teacher=Wte, b_teacher=bte)
    if head in ("ppo", "cispo"):
        tsub = dict(old_logprobs_rows=old[rows], clip_low=0.2, clip_high=0.28)
    sub = O.sampled_rows(X[rows], W, b, n_valid=full["n_valid"],
                         labels_rows=labels[rows],
                         target_rows=None if q is None else q[rows],
                         weights_rows=None if w is None else w[rows], **kw, **tsub)
    np.testing.assert_array_equal(sub["per_row"], full["per_row"][rows])
    np.testing.assert_allclose(sub["dX"], full["dX"][rows], rtol=1e-14, atol=1e-17)


# --------------------------------------------------------------------------
# cross-entropy head
# --------------------------------------------------------------------------

@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_ce_matches_torch_cross_entropy(reduction):
    X, W, b = _rand(12, 6), _rand(19, 6), _rand(19)
    y = rng.integers(0, 19, size=12)
    y[[2, 7]] = -100
    for tau in (0.5, 1.0):
        out = O.fwd_bwd(X, W, b, head="ce", labels=y, temperature=tau, reduction=reduction)
        ref = F.cross_entropy(torch.tensor(O.logits(X, W, b, tau)), torch.tensor(y),
                              ignore_index=-100, reduction=reduction)
        assert out["loss"] == pytest.approx(float(ref), rel=1e-13)
        assert (out["per_row"] >= 0).all()


def test_ce_weighted_matches_torch():
    X, W = _rand(10, 5), _rand(13, 5)
    y = rng.integers(0, 13, size=10)
    w = np.abs(_rand(10))
    out = O.fwd_bwd(X, W, head="ce", labels=y, weights=w, reduction="sum")
    ce = F.cross_entropy(torch.tensor(O.logits(X, W, None, 1.0)), torch.tensor(y),
                         reduction="none")
    assert out["loss"] == pytest.approx(float((torch.tensor(w) * ce).sum()), rel=1e-13)


def test_ce_equals_kl_with_one_hot_target():
    # cross-entropy is the KL head against a one-hot target (q log q = 0)
    X, W, b = _rand(9, 7), _rand(15, 7), _rand(15)
    y = rng.integers(0, 15, size=9)
    q = np.zeros((9, 15))
    q[np.arange(9), y] = 1.0
    for tau in (0.5, 2.0):
        a = O.fwd_bwd(X, W, b, head="ce", labels=y, temperature=tau, reduction="sum")
        c = O.fwd_bwd(X, W, b, head="kl", target=q, temperature=tau, reduction="sum")
        assert a["loss"] == pytest.approx(c["loss"], rel=1e-13)
        for k in ("dX", "dW", "db"):
            np.testing.assert_allclose(a[k], c[k], rtol=1e-12, atol=1e-15, err_msg=k)


# --------------------------------------------------------------------------
# Jensen-Shannon head (teacher with its own projection)
# --------------------------------------------------------------------------

def test_jsd_zero_when_teacher_is_the_student():
    # the same projection on both sides: P = Pt, so JS = 0 and every
    # student gradient vanishes
    X, W, b = _rand(11, 6), _rand(17, 6), _rand(17)
    out = O.fwd_bwd(X, W, b, head="jsd", X_teacher=X, W_teacher=W, b_teacher=b,
                    temperature=0.5, reduction="sum")
    assert abs(out["loss"]) <= 1e-15
    for k in ("dX", "dW", "db"):
        assert np.abs(out[k]).max() <= 1e-15, k


def test_jsd_matches_scipy_jensenshannon():
    # scipy's jensenshannon is the square root of the divergence (natural log)
    from scipy.spatial.distance import jensenshannon
    logP, _ = O.log_softmax(_rand(8, 23, std=2.0))
    Pt = _softmax(_rand(8, 23, std=2.0))
    ours = O.jsd_rows(logP, Pt, np.ones(8, bool))
    ref = np.array([jensenshannon(Pt[r], np.exp(logP[r])) ** 2 for r in range(8)])
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-15)


def test_jsd_bounds_and_symmetry():
    logP, _ = O.log_softmax(_rand(30, 40, std=4.0))
    logQ, _ = O.log_softmax(_rand(30, 40, std=4.0))
    a = O.jsd_rows(logP, np.exp(logQ), np.ones(30, bool))
    c = O.jsd_rows(logQ, np.exp(logP), np.ones(30, bool))
    np.testing.assert_allclose(a, c, rtol=1e-13)
    assert (a >= 0).all() and (a <= math.log(2) + 1e-15).all()


def test_jsd_disjoint_supports_is_log2():
    # no common support: M = P/2 on P's support and Q/2 on Q's, so each half
    # contributes log 2 / 2
    P = np.array([[0.5, 0.5, 0.0, 0.0], [0.0, 0.0, 0.0, 1.0]])
    Q = np.array([[0.0, 0.0, 0.3, 0.7], [0.2, 0.3, 0.5, 0.0]])
    with np.errstate(divide="ignore"):
        logQ = np.log(Q)
    L = O.jsd_rows(logQ, P, np.ones(2, bool))
    np.testing.assert_allclose(L, math.log(2), rtol=1e-15)


# --------------------------------------------------------------------------
# the row-blocked full pass (full-size parity of the GPU path)
# --------------------------------------------------------------------------

def _torch_logp_label(X, W, b, labels, tau):
    """log p(y_r) from torch's float64 log_softmax (0 where the label is
    ignored): an input builder independent of the oracle's own steps."""
    Z = F.linear(torch.tensor(X), torch.tensor(W), None if b is None else torch.tensor(b))
    logP = torch.log_softmax(Z / tau, dim=1).numpy()
    y = np.where(labels < 0, 0, labels)
    return np.where(labels < 0, 0.0, logP[np.arange(len(y)), y])


@pytest.mark.parametrize("head", ["kl", "selective", "ce", "jsd", "ppo", "cispo"])
def test_blocked_pass_equals_full(head):
    BT, H, V = 23, 8, 31
    X, W, b = _rand(BT, H), _rand(V, H), _rand(V)
    labels = rng.integers(0, V, size=BT)
    labels[[2, 11, 20]] = -100
    kw = dict(head=head, labels=labels, reduction="mean", temperature=2.0)
    if head == "kl":
        q = _softmax(_rand(BT, V))
        q[labels == -100] = np.nan  # never read
        kw["target"] = q
    elif head == "jsd":
        kw.update(X_teacher=_rand(BT, 5), W_teacher=_rand(V, 5), b_teacher=_rand(V))
    else:
        kw["weights"] = _rand(BT)
    if head in ("ppo", "cispo"):
        kw.update(old_logprobs=_torch_logp_label(X, W, b, labels, 2.0) - _rand(BT, std=0.3),
                  clip_low=0.2, clip_high=0.28)
    full = O.fwd_bwd(X, W, b, **kw)
    for block in (1, 5, 23, 64):  # ragged, one row, whole, larger than BT
        seen = []
        blk = O.fwd_bwd_blocked(X, W, b, block_rows=block, progress=lambda d, n: seen.append(d),
                                **kw)
        assert seen[-1] == BT
        assert blk["n_valid"] == full["n_valid"] and blk["g"] == full["g"]
        # BLAS may round a block's products differently from the whole
        # matrix's: agreement to a few ulps, not bitwise
        np.testing.assert_allclose(blk["per_row"], full["per_row"], rtol=1e-13, atol=1e-15)
        assert blk["loss"] == pytest.approx(full["loss"], rel=1e-13)
        for k in ("dX", "dW", "db"):
            np.testing.assert_allclose(blk[k], full[k], rtol=1e-13, atol=1e-15, err_msg=k)
    frozen = O.fwd_bwd_blocked(X, W, b, block_rows=4, compute_dW=False, compute_db=False,
                               **kw)
    assert frozen["dW"] is None and frozen["db"] is None


def test_blocked_pass_widens_float32_inputs():
    # float32 inputs (e.g. bf16 values) are widened exactly, block by block
    X = _rand(9, 8).astype(np.float32)
    W = _rand(19, 8).astype(np.float32)
    y = rng.integers(0, 19, size=9)
    a = O.fwd_bwd(X.astype(np.float64), W.astype(np.float64), head="ce", labels=y)
    c = O.fwd_bwd_blocked(X, W, head="ce", labels=y, block_rows=4)
    np.testing.assert_allclose(c["dW"], a["dW"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(c["dX"], a["dX"], rtol=1e-13, atol=1e-16)


# --------------------------------------------------------------------------
# KL: exact zeros in the target
# --------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 1e-10])
def test_kl_zero_target_entries_add_nothing_even_with_eps_zero(eps):
    # FusedLinearKLDivLoss page, Details: the clamp exists so that 0 log 0
    # contributes 0. One-hot targets make every entry but one exactly 0: the
    # KL is then the cross-entropy, for eps = 0 too.
    X, W, b, _ = _kl_case(BT=8, V=11)
    y = rng.integers(0, 11, size=8)
    q = np.zeros((8, 11))
    q[np.arange(8), y] = 1.0
    out = O.fwd_bwd(X, W, b, head="kl", target=q, reduction="sum", eps=eps)
    ce = F.cross_entropy(torch.tensor(O.logits(X, W, b, 1.0)), torch.tensor(y),
                         reduction="none")
    np.testing.assert_allclose(out["per_row"], ce.numpy(), rtol=1e-13)
    logP = torch.log_softmax(torch.tensor(O.logits(X, W, b, 1.0)), 1)
    ref = F.kl_div(logP, torch.tensor(q), reduction="sum")  # xlogy: 0 log 0 = 0
    assert out["loss"] == pytest.approx(float(ref), rel=1e-13)


def test_kl_eps_clamps_small_targets_inside_the_log():
    # 0 < q < eps: the term is q log(eps), not q log q
    logP, _ = O.log_softmax(np.array([[0.0, 1.0, 2.0]]))
    q = np.array([[1e-12, 0.5, 0.5 - 1e-12]])
    L = O.kl_rows(logP, q, np.ones(1, bool), 1e-6)
    ref = (1e-12 * math.log(1e-6) + 0.5 * math.log(0.5) + (0.5 - 1e-12) * math.log(0.5 - 1e-12)
           - (q[0] * logP[0]).sum())
    assert L[0] == pytest.approx(ref, rel=1e-14)


# --------------------------------------------------------------------------
# ratio heads: PPO clipped surrogate and CISPO
# --------------------------------------------------------------------------

# Two classes with logits [0, log 3]: p = [1/4, 3/4] exactly. Each row picks a
# label, a ratio rho (old = log p(y) - log rho) and an advantage A; the table
# gives the clipped-surrogate loss -min(rho A, clip(rho) A) and its derivative
# in log p(y) by hand, with clip range [1 - 0.2, 1 + 0.28].
PPO_TABLE = [
    # y, rho,  A,    loss,               dloss/dlogp
    (1, 1.0, 2.0, -2.0, -2.0),           # r = 1: unclipped, -A
    (0, 1.1, 2.0, -2.2, -2.2),           # inside the range
    (1, 1.25, 1.0, -1.25, -1.25),        # inside only with the wider upper clip
    (1, 1.5, 2.0, -2.56, 0.0),           # above, A > 0: clipped, no gradient
    (0, 0.5, 2.0, -1.0, -1.0),           # below, A > 0: unclipped rho A is smaller
    (1, 1.5, -1.0, 1.5, 1.5),            # above, A < 0: unclipped rho A is smaller
    (0, 0.5, -1.0, 0.8, 0.0),            # below, A < 0: clipped at 0.8, no gradient
    (1, 0.7, -3.0, 2.4, 0.0),            # below, A < 0
    (0, 3.0, 0.0, 0.0, 0.0),             # A = 0
]


def _two_class_rows(table):
    n = len(table)
    X = np.ones((n, 1))
    W = np.array([[0.0], [math.log(3.0)]])
    y = np.array([t[0] for t in table])
    logp = np.log(np.array([0.25, 0.75]))[y]
    old = logp - np.log(np.array([t[1] for t in table]))
    A = np.array([t[2] for t in table])
    return X, W, y, old, A


def test_ppo_closed_form_table():
    X, W, y, old, A = _two_class_rows(PPO_TABLE)
    out = O.fwd_bwd(X, W, head="ppo", labels=y, weights=A, old_logprobs=old,
                    clip_low=0.2, clip_high=0.28, reduction="sum")
    np.testing.assert_allclose(out["per_row"], [t[3] for t in PPO_TABLE], rtol=1e-13,
                               atol=1e-15)
    assert out["loss"] == pytest.approx(sum(t[3] for t in PPO_TABLE), rel=1e-13)
    # dZ_r = k_r (onehot(y_r) - p) with p = [1/4, 3/4]; dX_r = dZ_r W = k_r (d_y - 3/4) log 3
    k = np.array([t[4] for t in PPO_TABLE])
    dlogit1 = k * ((y == 1) - 0.75)
    np.testing.assert_allclose(out["dX"][:, 0], dlogit1 * math.log(3.0), rtol=1e-13,
                               atol=1e-15)
    np.testing.assert_allclose(out["db"], [-dlogit1.sum(), dlogit1.sum()], rtol=1e-12,
                               atol=1e-15)


def test_cispo_closed_form_table():
    X, W, y, old, A = _two_class_rows(PPO_TABLE)
    out = O.fwd_bwd(X, W, head="cispo", labels=y, weights=A, old_logprobs=old,
                    clip_low=0.2, clip_high=0.28, reduction="sum")
    c = np.clip([t[1] for t in PPO_TABLE], 0.8, 1.28)
    logp = np.log(np.array([0.25, 0.75]))[y]
    np.testing.assert_allclose(out["per_row"], -c * A * logp, rtol=1e-13, atol=1e-15)
    dlogit1 = -c * A * ((y == 1) - 0.75)
    np.testing.assert_allclose(out["dX"][:, 0], dlogit1 * math.log(3.0), rtol=1e-13,
                               atol=1e-15)


def _ratio_case(BT=13, H=6, V=17, tau=2.0, spread=0.3, seed_shift=0.0):
    X, W, b = _rand(BT, H), _rand(V, H), _rand(V)
    labels = rng.integers(0, V, size=BT)
    labels[[1, 8]] = -100
    A = _rand(BT)
    # log-ratios away from the clip boundaries log(0.8) and log(1.28), so a
    # finite-difference step never crosses one
    d = _rand(BT, std=spread) + seed_shift
    for edge in (math.log(0.8), math.log(1.28)):
        near = np.abs(d - edge) < 0.02
        d[near] += 0.05
    old = _torch_logp_label(X, W, b, labels, tau) - d
    return X, W, b, labels, A, old, d


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_ppo_and_cispo_at_ratio_one_are_the_selective_head(reduction):
    # old = new log-probs: rho = 1 everywhere, so PPO's gradient is that of
    # the selective head with weights -A, and CISPO (weight clip(1) = 1) is
    # that head with weights -A in loss and gradients
    X, W, b, labels, A, _, _ = _ratio_case()
    old = _torch_logp_label(X, W, b, labels, 2.0)
    sel = O.fwd_bwd(X, W, b, head="selective", labels=labels, weights=-A, temperature=2.0,
                    reduction=reduction)
    for head in ("ppo", "cispo"):
        out = O.fwd_bwd(X, W, b, head=head, labels=labels, weights=A, old_logprobs=old,
                        temperature=2.0, reduction=reduction)
        for k in ("dX", "dW", "db"):
            np.testing.assert_allclose(out[k], sel[k], rtol=1e-12, atol=1e-15, err_msg=k)
    ppo = O.fwd_bwd(X, W, b, head="ppo", labels=labels, weights=A, old_logprobs=old,
                    temperature=2.0, reduction=reduction)
    keep = labels != -100
    g = 1.0 if reduction == "sum" else 1.0 / keep.sum()
    assert ppo["loss"] == pytest.approx(-g * A[keep].sum(), rel=1e-12)
    cis = O.fwd_bwd(X, W, b, head="cispo", labels=labels, weights=A, old_logprobs=old,
                    temperature=2.0, reduction=reduction)
    assert cis["loss"] == pytest.approx(sel["loss"], rel=1e-12)


def _torch_ratio_loss(head, X, W, b, labels, A, old, tau, lo, hi, reduction):
    Xt, Wt, bt = (torch.tensor(a, requires_grad=True) for a in (X, W, b))
    logP = torch.log_softmax(F.linear(Xt, Wt, bt) / tau, dim=1)
    keep = torch.tensor(labels != -100)
    y = torch.tensor(np.where(labels < 0, 0, labels))
    lp = logP[torch.arange(len(labels)), y]
    rho = torch.exp(lp - torch.tensor(old))
    At = torch.tensor(A)
    c = torch.clamp(rho, 1 - lo, 1 + hi)
    if head == "ppo":
        per = -torch.minimum(rho * At, c * At)
    else:
        per = -c.detach() * At * lp
    loss = per[keep].sum()
    if reduction != "sum":
        loss = loss / keep.sum()
    loss.backward()
    return loss, per.detach(), Xt.grad, Wt.grad, bt.grad


@pytest.mark.parametrize("head", ["ppo", "cispo"])
@pytest.mark.parametrize("lo,hi", [(0.2, 0.28), (0.1, 0.1), (1.0, 1e300)])
def test_ratio_heads_match_torch_autograd(head, lo, hi):
    # (1.0, 1e300): no clipping at all, the plain ratio objective -rho A
    X, W, b, labels, A, old, d = _ratio_case(BT=40, spread=0.5)
    if (lo, hi) == (0.1, 0.1):
        for edge in (math.log(0.9), math.log(1.1)):
            d2 = np.log(np.exp(_torch_logp_label(X, W, b, labels, 2.0) - old))
            assert (np.abs(d2 - edge) > 1e-6).all()
    loss, per, gX, gW, gb = _torch_ratio_loss(head, X, W, b, labels, A, old, 2.0, lo, hi,
                                              "mean")
    out = O.fwd_bwd(X, W, b, head=head, labels=labels, weights=A, old_logprobs=old,
                    clip_low=lo, clip_high=hi, temperature=2.0, reduction="mean")
    assert out["loss"] == pytest.approx(float(loss), rel=1e-12)
    keep = labels != -100
    np.testing.assert_allclose(out["per_row"][keep], per.numpy()[keep], rtol=1e-12)
    np.testing.assert_allclose(out["dX"], gX.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["dW"], gW.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["db"], gb.numpy(), rtol=1e-10, atol=1e-14)
    if hi == 1e300 and head == "ppo":
        assert (out["per_row"][keep] == pytest.approx(
            -np.exp(d[keep]) * A[keep], rel=1e-12))


def test_ppo_both_branches_are_exercised():
    _, _, _, labels, A, _, d = _ratio_case(BT=40, spread=0.5)
    rho = np.exp(d)
    keep = labels != -100
    clipped = keep & (rho * A > np.clip(rho, 0.8, 1.28) * A)
    assert 0 < clipped.sum() < keep.sum()


@pytest.mark.parametrize("tau", [0.5, 2.0])
def test_ppo_gradients_central_differences(tau):
    BT, H, V = 6, 4, 7
    X, W, b = _rand(BT, H), _rand(V, H), _rand(V)
    labels = rng.integers(0, V, size=BT)
    labels[2] = -100
    A = _rand(BT)
    d = np.array([0.0, 0.5, 0.0, -0.6, 0.1, -0.1])  # both branches and the interior
    old = _torch_logp_label(X, W, b, labels, tau) - d
    kw = dict(head="ppo", labels=labels, weights=A, old_logprobs=old, clip_low=0.2,
              clip_high=0.28, temperature=tau, reduction="mean")
    out = O.fwd_bwd(X, W, b, **kw)
    f = _loss_fn(kw)
    for i, name in ((0, "dX"), (1, "dW"), (2, "db")):
        fd = _central_fd(f, [X, W, b], i)
        np.testing.assert_allclose(out[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_cispo_gradient_is_the_frozen_weight_surrogate():
    # with sg(c) the gradient is that of -c0 A log p(y) for c0 fixed at the
    # current point: finite differences of that surrogate
    BT, H, V, tau = 6, 4, 7, 1.0
    X, W, b = _rand(BT, H), _rand(V, H), _rand(V)
    labels = rng.integers(0, V, size=BT)
    A = _rand(BT)
    d = np.array([0.0, 0.5, 0.1, -0.6, 0.1, -0.1])
    old = _torch_logp_label(X, W, b, labels, tau) - d
    c0 = np.clip(np.exp(d), 0.8, 1.28)
    out = O.fwd_bwd(X, W, b, head="cispo", labels=labels, weights=A, old_logprobs=old,
                    clip_low=0.2, clip_high=0.28, temperature=tau, reduction="sum")

    def surrogate(X_, W_, b_):
        lp = _torch_logp_label(X_, W_, b_, labels, tau)
        return float(-(c0 * A * lp).sum())

    for i, name in ((0, "dX"), (1, "dW"), (2, "db")):
        fd = _central_fd(surrogate, [X, W, b], i)
        np.testing.assert_allclose(out[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("head", ["ppo", "cispo"])
def test_ratio_heads_scale_with_positive_advantage_factor(head):
    # a positive per-token factor (GRPO's 1/|o_i|, Dr. GRPO's constant) folds
    # into A: loss and gradients scale by it, the clip decisions do not move
    X, W, b, labels, A, old, _ = _ratio_case()
    a = O.fwd_bwd(X, W, b, head=head, labels=labels, weights=A, old_logprobs=old,
                  temperature=2.0, reduction="sum")
    c = O.fwd_bwd(X, W, b, head=head, labels=labels, weights=4.0 * A, old_logprobs=old,
                  temperature=2.0, reduction="sum")
    assert c["loss"] == pytest.approx(4.0 * a["loss"], rel=1e-13)
    for k in ("dX", "dW", "db"):
        np.testing.assert_allclose(c[k], 4.0 * a[k], rtol=1e-13, atol=1e-16, err_msg=k)


@pytest.mark.parametrize("head", ["ppo", "cispo"])
def test_ratio_heads_dlogit_rows_sum_to_zero_and_tau_identity(head):
    X, W, b, labels, A, old, _ = _ratio_case(H=8)
    out = O.fwd_bwd(X, W, b, head=head, labels=labels, weights=A, old_logprobs=old,
                    temperature=2.0, reduction="sum")
    np.testing.assert_allclose(out["db"].sum(), 0.0, atol=1e-14)
    # tau = 2: (X W^T + b) / 2 = X (W/2)^T + b/2 exactly
    c = O.fwd_bwd(X, W / 2, b / 2, head=head, labels=labels, weights=A, old_logprobs=old,
                  temperature=1.0, reduction="sum")
    assert out["loss"] == c["loss"]
    np.testing.assert_array_equal(out["dX"], c["dX"])
    np.testing.assert_array_equal(out["dW"], c["dW"] / 2)


def test_ratio_heads_need_old_logprobs():
    with pytest.raises(ValueError):
        O.fwd_bwd(_rand(2, 3), _rand(4, 3), head="ppo", labels=np.array([0, 1]))


def test_label_logprobs_is_the_selective_log_prob():
    X, W, b = _rand(11, 5), _rand(23, 5), _rand(23)
    y = rng.integers(0, 23, size=11)
    y[4] = -100
    lp = O.label_logprobs(X, W, b, y, temperature=0.5, block_rows=3)
    np.testing.assert_allclose(lp, _torch_logp_label(X, W, b, y, 0.5), rtol=1e-13)
    assert lp[4] == 0.0
