"""CPU float64 oracle for the fused lm_head loss with gradient-in-forward.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, materialised
definition of what the HIP path computes. Only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it. The product path never calls it, and it shares no code with the HIP
path: it imports numpy and nothing else.

Pages cited (titles as used throughout this repository):

* "FusedLinearKLDivLoss page" -- the Liger-Kernel pull request that adds
  ``FusedLinearKLDivLoss`` (sections Summary, Details, Testing Done).
* "frozen lm_head GRPO page" -- the Liger-Kernel pull request that stops
  ``_ChunkedSelectiveLogProbFunction`` from forming the lm_head gradient
  when the head is frozen (sections Summary, Details, Testing Done).
* "LoRA normalization page" -- the Liger-Kernel pull request that adds
  ``COMPUTE_DW`` / ``COMPUTE_DB`` to the norm backward kernels (sections
  Motivation, Key Changes, Test Validation).

What is computed, for every token row r of X [BT, H] against the head
W [V, H] (+ b [V]):

1. logits Z = X W^T + b, tempered S = Z / tau (model side only).
2. log-softmax over the vocabulary: logP = S - lse(S).
3. the per-row term of one of three heads:
   KL:        L_r = sum_v q_rv * log(max(q_rv, eps)) - q_rv * logP_rv
   SELECTIVE: L_r = logP_{r, y_r}   (weighted by the advantage w_r)
   CE:        L_r = -logP_{r, y_r}  (cross-entropy: KL against a one-hot target)
4. loss = g * sum_r w_r L_r with g from the reduction and the count of rows
   whose label is not ``ignore_index``.
5. the exact gradient: dS = d loss / d S, dZ = dS / tau, then
   dX = dZ W, dW = dZ^T X, db = sum_r dZ_r.

Readings of points the pages leave open (each repeated where it is used):
KL direction is KL(target || model); eps clamps q inside the log only;
the temperature divides the model logits only, with no tau^2 factor;
ignored rows leave the batch (denominators count valid rows only);
the selective head's loss is the advantage-weighted mean of log p(label),
not negated; "mean" and "batchmean" coincide for the selective head.

Parity status: every function below is pinned by the CPU tests against
closed forms, invariants, torch library routines in float64 and central
finite differences. The *choices* of the readings listed above (eps value,
denominator with ignored rows, sign and normaliser of the selective head)
are fixed by reading, not by a number the pages print.
"""

from __future__ import annotations

import numpy as np

HEAD_KL = "kl"
HEAD_SELECTIVE = "selective"
HEAD_CE = "ce"
REDUCTIONS = ("batchmean", "mean", "sum")


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def logits(X, W, b, temperature):
    """Tempered logits S = (X W^T + b) / tau, fully materialised.

    FusedLinearKLDivLoss page, Summary: the loss fuses the vocabulary-head
    linear projection; Details: a softmax ``temperature`` is applied. The
    temperature divides the model logits only (the target is an explicit
    distribution and is not re-tempered; no tau^2 factor is mentioned).
    """
    Z = _f64(X) @ _f64(W).T
    if b is not None:
        Z = Z + _f64(b)[None, :]
    return Z / float(temperature)


def log_softmax(S):
    """Row log-softmax over the vocabulary: logP = S - (m + log sum exp(S - m)).

    Returns (logP, lse). The max m is only a stabiliser: any row maximum gives
    the same lse. FusedLinearKLDivLoss page, Details (log-softmax and its
    backward on the saved log-probs).
    """
    m = S.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(S - m).sum(axis=1, keepdims=True))
    return S - lse, lse[:, 0]


def valid_rows(labels, ignore_index, BT):
    """Rows that take part in the loss.

    FusedLinearKLDivLoss page, Details: ``ignore_index`` via ``shift_labels``.
    For the KL head the labels act only as a row mask; with no labels every
    row is valid.
    """
    if labels is None:
        return np.ones(BT, dtype=bool)
    return np.asarray(labels) != ignore_index


def kl_rows(logP, target, valid, eps):
    """Per-row KL(target || model) = sum_v q log(max(q, eps)) - q logP.

    FusedLinearKLDivLoss page, Summary: KL(Q || P) against an explicit target
    distribution; Details: an ``eps`` clamp so that 0 * log(0) contributes 0
    (read as a clamp of q inside the log only, so q = 0 gives exactly 0).
    Ignored rows give 0 and their targets are never read.
    """
    L = np.zeros(logP.shape[0])
    r = np.nonzero(valid)[0]
    if r.size:
        q = _f64(target)[r]
        L[r] = (q * np.log(np.maximum(q, eps)) - q * logP[r]).sum(axis=1)
    return L


def ce_rows(logP, labels, valid):
    """Per-row cross-entropy -log p(y_r): the KL head with a one-hot target
    (q log q vanishes), the fused linear cross-entropy head the
    FusedLinearKLDivLoss page (Summary) takes its chunk geometry from."""
    return -selective_rows(logP, labels, valid)


def selective_rows(logP, labels, valid):
    """Per-row selective log-prob log p(y_r) of the label.

    frozen lm_head GRPO page, Summary: ``_ChunkedSelectiveLogProbFunction``
    forms per-token log-probabilities of the chosen tokens. Ignored rows give 0.
    """
    L = np.zeros(logP.shape[0])
    r = np.nonzero(valid)[0]
    if r.size:
        y = np.asarray(labels)[r]
        if np.any((y < 0) | (y >= logP.shape[1])):
            raise ValueError("label outside [0, V) on a non-ignored row")
        L[r] = logP[r, y]
    return L


def reduction_scale(head, reduction, n_valid, V):
    """The factor g with loss = g * sum_r w_r L_r.

    FusedLinearKLDivLoss page, Details: reductions batchmean / mean / sum with
    the semantics of ``torch.nn.KLDivLoss`` (batchmean divides by the batch,
    mean by the element count, sum by 1); ``"none"`` is refused because
    gradient-in-forward needs a scalar loss. With ignored rows the batch is the
    valid rows. For the selective and cross-entropy heads the tokens are the
    batch, so mean and batchmean both divide by the valid-token count (the
    ``torch.nn.functional.cross_entropy`` mean with ``ignore_index``). No valid
    row gives g = 0.
    """
    if reduction not in REDUCTIONS:
        raise ValueError(f"unsupported reduction {reduction!r}")
    if n_valid == 0:
        return 0.0
    if reduction == "sum":
        return 1.0
    if reduction == "mean" and head == HEAD_KL:
        return 1.0 / (n_valid * V)
    return 1.0 / n_valid


def row_weights(head, weights, BT):
    """Per-row loss weights: the advantages of the selective head (optional
    per-token weights of the cross-entropy head), else 1."""
    if head in (HEAD_SELECTIVE, HEAD_CE) and weights is not None:
        return _f64(weights)
    return np.ones(BT)


def dlogits(head, logP, target, labels, w, valid, g, temperature):
    """Exact gradient of the loss with respect to the raw logits Z.

    With P = exp(logP) and S = Z / tau:
      KL:        dS_r = g * (Q_r * P_r - q_r),   Q_r = sum_v q_rv
      SELECTIVE: dS_r = g * w_r * (onehot(y_r) - P_r)
      CE:        dS_r = g * w_r * (P_r - onehot(y_r))
    and dZ = dS / tau. Ignored rows are 0. This is the log-softmax backward
    the FusedLinearKLDivLoss page (Details) computes in place on the saved
    log-probs; Q_r keeps it exact even when a target row does not sum to 1.
    """
    BT, V = logP.shape
    dS = np.zeros((BT, V))
    r = np.nonzero(valid)[0]
    if r.size:
        P = np.exp(logP[r])
        if head == HEAD_KL:
            q = _f64(target)[r]
            Q = q.sum(axis=1, keepdims=True)
            dS[r] = g * (Q * P - q)
        else:
            y = np.asarray(labels)[r]
            onehot = np.zeros_like(P)
            onehot[np.arange(r.size), y] = 1.0
            sign = -1.0 if head == HEAD_CE else 1.0
            dS[r] = sign * g * w[r][:, None] * (onehot - P)
    return dS / float(temperature)


def fwd_bwd(X, W, b=None, *, head, labels=None, target=None, weights=None,
            reduction="batchmean", ignore_index=-100, temperature=1.0,
            eps=1e-10, compute_dW=True, compute_db=True):
    """Loss and gradients of the fused lm_head loss, fully materialised.

    The chunked gradient-in-forward structure (FusedLinearKLDivLoss page,
    Summary) reaches this same result without forming the BT x V logits; the
    oracle forms them. dX is always produced; dW = dZ^T X and db = sum_r dZ_r
    only when asked for (frozen lm_head GRPO page, Summary: only the gradients
    autograd asks for; LoRA normalization page, Key Changes: COMPUTE_DW and
    COMPUTE_DB prune weight and bias gradients independently).

    Returns a dict with loss (float), per_row [BT] (KL_r, log p(y_r) or
    -log p(y_r); 0 on ignored rows), dX [BT, H], dW [V, H] or None, db [V] or None, n_valid, g.
    """
    if head not in (HEAD_KL, HEAD_SELECTIVE, HEAD_CE):
        raise ValueError(f"unknown head {head!r}")
    if not (temperature > 0 and np.isfinite(temperature)):
        raise ValueError("temperature must be positive and finite")
    X = _f64(X)
    W = _f64(W)
    BT, H = X.shape
    V = W.shape[0]
    valid = valid_rows(labels, ignore_index, BT)
    n_valid = int(valid.sum())
    g = reduction_scale(head, reduction, n_valid, V)
    w = row_weights(head, weights, BT)

    S = logits(X, W, b, temperature)
    logP, _ = log_softmax(S)
    del S
    if head == HEAD_KL:
        if target is None:
            raise ValueError("the KL head needs a target distribution")
        L = kl_rows(logP, target, valid, eps)
    else:
        if labels is None:
            raise ValueError("the selective and cross-entropy heads need labels")
        L = (ce_rows if head == HEAD_CE else selective_rows)(logP, labels, valid)
    loss = g * float((w * L).sum())

    dZ = dlogits(head, logP, target, labels, w, valid, g, temperature)
    del logP
    out = dict(loss=loss, per_row=L, n_valid=n_valid, g=g, dW=None, db=None)
    out["dX"] = dZ @ W
    if compute_dW:
        out["dW"] = dZ.T @ X
    if compute_db:
        out["db"] = dZ.sum(axis=0)
    return out


def sampled_rows(X_rows, W, b=None, *, head, n_valid, labels_rows=None,
                 target_rows=None, weights_rows=None, reduction="batchmean",
                 ignore_index=-100, temperature=1.0, eps=1e-10):
    """The same definition restricted to a subset of rows.

    Every step above except the final reduction is row-local, so for a subset
    of rows the per-row terms and the dX rows follow from the rows themselves
    and the global valid-row count ``n_valid`` (which fixes g). Used to check
    full-size runs whose BT x V logits the oracle cannot form in seconds.

    Returns a dict with per_row [R], weighted [R] = g * w_r * L_r (the rows'
    share of the loss) and dX [R, H].
    """
    X_rows = _f64(X_rows)
    W = _f64(W)
    R = X_rows.shape[0]
    V = W.shape[0]
    valid = valid_rows(labels_rows, ignore_index, R)
    g = reduction_scale(head, reduction, n_valid, V)
    w = row_weights(head, weights_rows, R)
    S = logits(X_rows, W, b, temperature)
    logP, _ = log_softmax(S)
    if head == HEAD_KL:
        L = kl_rows(logP, target_rows, valid, eps)
    elif head == HEAD_CE:
        L = ce_rows(logP, labels_rows, valid)
    else:
        L = selective_rows(logP, labels_rows, valid)
    dZ = dlogits(head, logP, target_rows, labels_rows, w, valid, g, temperature)
    return dict(per_row=L, weighted=g * w * L, dX=dZ @ W, g=g)
