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
3. the per-row term of one of four heads:
   KL:        L_r = sum_v q_rv * log(max(q_rv, eps)) - q_rv * logP_rv
   SELECTIVE: L_r = logP_{r, y_r}   (weighted by the advantage w_r)
   CE:        L_r = -logP_{r, y_r}  (cross-entropy: KL against a one-hot target)
   JSD:       L_r = 1/2 KL(Pt_r || M_r) + 1/2 KL(P_r || M_r), M = (Pt + P) / 2,
              Pt = softmax of a teacher's own tempered logits
              (X_t W_t^T + b_t) / tau, the teacher taking no gradient
   PPO:       L_r = -min(rho_r A_r, clip(rho_r, 1 - e_lo, 1 + e_hi) A_r),
              rho_r = exp(logP_{r, y_r} - old_r)  (clipped surrogate)
   CISPO:     L_r = -sg(clip(rho_r, 1 - e_lo, 1 + e_hi)) A_r logP_{r, y_r}
              (clipped importance weight, no gradient through it)
4. loss = g * sum_r w_r L_r with g from the reduction and the count of rows
   whose label is not ``ignore_index``.
5. the exact gradient: dS = d loss / d S, dZ = dS / tau, then
   dX = dZ W, dW = dZ^T X, db = sum_r dZ_r.

Readings of points the pages leave open (each repeated where it is used):
KL direction is KL(target || model); eps clamps q inside the log only;
the temperature divides the model logits only, with no tau^2 factor;
ignored rows leave the batch (denominators count valid rows only);
the selective head's loss is the advantage-weighted mean of log p(label),
not negated; "mean" and "batchmean" coincide for the selective head;
the JSD head is the symmetric Jensen-Shannon divergence in natural log, the
temperature dividing both the teacher's and the student's logits; the ratio
heads take the published PPO clipped surrogate (Schulman et al., 2017, with
DAPO's separate lower and upper clip widths) and CISPO's clipped,
gradient-free importance weight (MiniMax-M1 report, 2025) as the plainest
members of the family the frozen lm_head GRPO page names, written as losses
to minimise; a tie between the unclipped and clipped products takes the
unclipped branch.

Parity status: every function below is pinned by the CPU tests against
closed forms, invariants, torch library routines in float64 and central
finite differences. The *choices* of the readings listed above (eps value,
denominator with ignored rows, sign and normaliser of the selective head,
which members of the GRPO family the ratio heads take) are fixed by reading,
not by a number the pages print: parity unpinned for those choices.
"""

from __future__ import annotations

import numpy as np

HEAD_KL = "kl"
HEAD_SELECTIVE = "selective"
HEAD_CE = "ce"
HEAD_JSD = "jsd"
HEAD_PPO = "ppo"
HEAD_CISPO = "cispo"
LABEL_HEADS = (HEAD_SELECTIVE, HEAD_CE, HEAD_PPO, HEAD_CISPO)
RATIO_HEADS = (HEAD_PPO, HEAD_CISPO)
HEADS = (HEAD_KL, HEAD_SELECTIVE, HEAD_CE, HEAD_JSD, HEAD_PPO, HEAD_CISPO)
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
    (read as a clamp of q inside the log only). An entry with q = 0 adds
    exactly 0 whatever eps is, eps = 0 included: that is the stated purpose
    of the clamp. Ignored rows give 0 and their targets are never read.
    """
    L = np.zeros(logP.shape[0])
    r = np.nonzero(valid)[0]
    if r.size:
        q = _f64(target)[r]
        with np.errstate(divide="ignore", invalid="ignore"):
            qlogq = np.where(q > 0, q * np.log(np.maximum(q, eps)), 0.0)
        L[r] = (qlogq - q * logP[r]).sum(axis=1)
    return L


def jsd_rows(logP, teacher, valid):
    """Per-row Jensen-Shannon divergence between the teacher distribution
    Pt (``teacher``, probabilities) and the model P = exp(logP):

        JS_r = 1/2 sum_v Pt log(Pt / M) + 1/2 sum_v P log(P / M),  M = (Pt + P) / 2,

    natural log, a zero probability contributing 0. FusedLinearKLDivLoss
    page, Summary: the fused JSD loss whose teacher side has its own
    projection (the divergence itself is not printed there; the symmetric
    Jensen-Shannon divergence is the plain reading). Ignored rows give 0.
    """
    L = np.zeros(logP.shape[0])
    r = np.nonzero(valid)[0]
    if r.size:
        Pt = _f64(teacher)[r]
        P = np.exp(logP[r])
        M = 0.5 * (Pt + P)
        with np.errstate(divide="ignore", invalid="ignore"):
            tt = np.where(Pt > 0, Pt * np.log(Pt / M), 0.0)
            tp = np.where(P > 0, P * np.log(P / M), 0.0)
        L[r] = 0.5 * (tt.sum(axis=1) + tp.sum(axis=1))
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


def label_logprobs(X, W, b, labels, *, temperature=1.0, ignore_index=-100,
                   block_rows=512):
    """log p(y_r) of every row's label, 0 on ignored rows: the selective
    log-prob alone (frozen lm_head GRPO page, Summary), formed block by block
    so any batch fits in host memory. The tests of the ratio heads form their
    old log-probs from it."""
    W = _f64(W)
    BT = X.shape[0]
    out = np.zeros(BT)
    valid = valid_rows(labels, ignore_index, BT)
    for r0 in range(0, BT, block_rows):
        rows = slice(r0, min(BT, r0 + block_rows))
        logP, _ = log_softmax(logits(_f64(X[rows]), W, b, temperature))
        out[rows] = selective_rows(logP, labels[rows], valid[rows])
    return out


def ratio_rows(head, logP, labels, valid, old_logprobs, advantages, clip_low, clip_high):
    """Per-row loss L_r and its derivative k_r = dL_r / d logP_{r, y_r} for
    the ratio heads, on top of the selective log-prob of the label.

    frozen lm_head GRPO page, Summary: the GRPO loss family (GRPO, DAPO,
    Dr. GRPO, BNPO, CISPO, SAPO) is built on the chunked selective log-prob;
    the page prints no formula, so the published definitions are taken:

    * PPO clipped surrogate (Schulman et al., 2017), with the separate lower
      and upper clip widths of DAPO's "clip-higher":
        rho = exp(logP_y - old),  c = clip(rho, 1 - clip_low, 1 + clip_high)
        L = -min(rho A, c A)
        k = -rho A where rho A <= c A (the unclipped product is the minimum;
            a tie, e.g. inside the clip range, takes this branch), else 0
            (the clipped product is constant in logP_y).
    * CISPO (MiniMax-M1 report, 2025): the clipped ratio is a weight with no
      gradient through it:
        L = -sg(c) A logP_y,  k = -c A.

    Both are losses to minimise (the module the page describes is a loss).
    GRPO's per-sequence mean and Dr. GRPO's constant normaliser are positive
    per-token factors, so they fold into A with reduction "sum"; DAPO's and
    BNPO's token mean is reduction "mean". Ignored rows give L = k = 0.
    """
    BT = logP.shape[0]
    L = np.zeros(BT)
    k = np.zeros(BT)
    r = np.nonzero(valid)[0]
    if r.size:
        lp = selective_rows(logP, labels, valid)[r]
        A = np.ones(r.size) if advantages is None else _f64(advantages)[r]
        rho = np.exp(lp - _f64(old_logprobs)[r])
        c = np.clip(rho, 1.0 - clip_low, 1.0 + clip_high)
        if head == HEAD_PPO:
            unclipped, clipped = rho * A, c * A
            L[r] = -np.minimum(unclipped, clipped)
            k[r] = np.where(unclipped <= clipped, -rho * A, 0.0)
        elif head == HEAD_CISPO:
            L[r] = -c * A * lp
            k[r] = -c * A
        else:
            raise ValueError(f"{head!r} is not a ratio head")
    return L, k


def reduction_scale(head, reduction, n_valid, V):
    """The factor g with loss = g * sum_r w_r L_r.

    FusedLinearKLDivLoss page, Details: reductions batchmean / mean / sum with
    the semantics of ``torch.nn.KLDivLoss`` (batchmean divides by the batch,
    mean by the element count, sum by 1); ``"none"`` is refused because
    gradient-in-forward needs a scalar loss. With ignored rows the batch is the
    valid rows; the JSD head, a divergence between distributions like KL,
    takes KL's semantics. For the label heads (selective, cross-entropy and
    the ratio heads) the tokens are the batch, so mean and batchmean both
    divide by the valid-token count (the ``torch.nn.functional.cross_entropy``
    mean with ``ignore_index``; the token mean of DAPO and BNPO). No valid
    row gives g = 0.
    """
    if reduction not in REDUCTIONS:
        raise ValueError(f"unsupported reduction {reduction!r}")
    if n_valid == 0:
        return 0.0
    if reduction == "sum":
        return 1.0
    if reduction == "mean" and head in (HEAD_KL, HEAD_JSD):
        return 1.0 / (n_valid * V)
    return 1.0 / n_valid


def row_weights(head, weights, BT):
    """Per-row loss weights: the advantages of the selective head (optional
    per-token weights of the cross-entropy head), else 1. The ratio heads
    take their advantages inside the per-row term, so their weight is 1."""
    if head in (HEAD_SELECTIVE, HEAD_CE) and weights is not None:
        return _f64(weights)
    return np.ones(BT)


def dlogits(head, logP, target, labels, w, valid, g, temperature):
    """Exact gradient of the loss with respect to the raw logits Z.

    With P = exp(logP) and S = Z / tau:
      KL:        dS_r = g * (Q_r * P_r - q_r),   Q_r = sum_v q_rv
      SELECTIVE: dS_r = g * w_r * (onehot(y_r) - P_r)
      CE:        dS_r = g * w_r * (P_r - onehot(y_r))
      JSD:       dS_r = g * P_r * (G_r - sum_v P_rv G_rv),  G = 1/2 log(P / M)
      PPO/CISPO: dS_r = g * w_r * (onehot(y_r) - P_r) with w_r = k_r, the
                 derivative of the row's term in log p(y_r) (``ratio_rows``)
    and dZ = dS / tau. Ignored rows are 0. This is the log-softmax backward
    the FusedLinearKLDivLoss page (Details) computes in place on the saved
    log-probs; Q_r keeps it exact even when a target row does not sum to 1.
    For JSD (``target`` = the teacher probabilities Pt, M = (Pt + P) / 2):
    d JS / dP_v = 1/2 log(P_v / M_v) (the Pt / M and P / M terms of the
    derivative of M cancel to a constant that the softmax Jacobian removes),
    then the softmax Jacobian gives P_v (G_v - sum_u P_u G_u); G_v is taken
    as 0 where P_v = 0, its limit in the product.
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
        elif head == HEAD_JSD:
            Pt = _f64(target)[r]
            M = 0.5 * (Pt + P)
            with np.errstate(divide="ignore", invalid="ignore"):
                G = np.where(P > 0, 0.5 * np.log(P / M), 0.0)
            dS[r] = g * P * (G - (P * G).sum(axis=1, keepdims=True))
        else:
            y = np.asarray(labels)[r]
            onehot = np.zeros_like(P)
            onehot[np.arange(r.size), y] = 1.0
            sign = -1.0 if head == HEAD_CE else 1.0
            dS[r] = sign * g * w[r][:, None] * (onehot - P)
    return dS / float(temperature)


def teacher_probs(X_teacher, W_teacher, b_teacher, temperature):
    """The JSD head's teacher distribution: softmax of the teacher's own
    tempered logits (X_t W_t^T + b_t) / tau (FusedLinearKLDivLoss page,
    Summary: the JSD teacher side needs its own projection)."""
    logPt, _ = log_softmax(logits(X_teacher, W_teacher, b_teacher, temperature))
    return np.exp(logPt)


def _check_head(head, temperature):
    if head not in HEADS:
        raise ValueError(f"unknown head {head!r}")
    if not (temperature > 0 and np.isfinite(temperature)):
        raise ValueError("temperature must be positive and finite")


def _rows(head, X, W, b, *, labels, target, weights, valid, g, temperature, eps,
          X_teacher, W_teacher, b_teacher, old_logprobs, clip_low, clip_high):
    """Steps 1-3 and the dlogits for a set of rows (every step is row-local
    once g is known): returns the per-row terms L, their loss weights and
    dZ = dS / tau, each for exactly these rows."""
    R = X.shape[0]
    S = logits(X, W, b, temperature)
    logP, _ = log_softmax(S)
    del S
    w = row_weights(head, weights, R)
    wgrad = w
    if head == HEAD_KL:
        if target is None:
            raise ValueError("the KL head needs a target distribution")
        L = kl_rows(logP, target, valid, eps)
    elif head == HEAD_JSD:
        if X_teacher is None or W_teacher is None or target is not None:
            raise ValueError("the JSD head needs a teacher projection and no target")
        target = teacher_probs(X_teacher, W_teacher, b_teacher, temperature)
        L = jsd_rows(logP, target, valid)
    else:
        if labels is None:
            raise ValueError("the label heads need labels")
        if head in RATIO_HEADS:
            if old_logprobs is None:
                raise ValueError("the ratio heads need the old log-probs")
            L, wgrad = ratio_rows(head, logP, labels, valid, old_logprobs, weights,
                                  clip_low, clip_high)
        else:
            L = (ce_rows if head == HEAD_CE else selective_rows)(logP, labels, valid)
    dZ = dlogits(head, logP, target, labels, wgrad, valid, g, temperature)
    return L, w, dZ


def fwd_bwd(X, W, b=None, *, head, labels=None, target=None, weights=None,
            reduction="batchmean", ignore_index=-100, temperature=1.0,
            eps=1e-10, compute_dW=True, compute_db=True, X_teacher=None,
            W_teacher=None, b_teacher=None, old_logprobs=None, clip_low=0.2,
            clip_high=0.2):
    """Loss and gradients of the fused lm_head loss, fully materialised.

    The chunked gradient-in-forward structure (FusedLinearKLDivLoss page,
    Summary) reaches this same result without forming the BT x V logits; the
    oracle forms them. dX is always produced; dW = dZ^T X and db = sum_r dZ_r
    only when asked for (frozen lm_head GRPO page, Summary: only the gradients
    autograd asks for; LoRA normalization page, Key Changes: COMPUTE_DW and
    COMPUTE_DB prune weight and bias gradients independently).

    Returns a dict with loss (float), per_row [BT] (KL_r, log p(y_r),
    -log p(y_r), JS_r or the ratio heads' L_r; 0 on ignored rows), dX [BT, H],
    dW [V, H] or None, db [V] or None, n_valid, g, and dZ [BT, V], the
    gradient with respect to the raw logits (dX = dZ W, dW = dZ^T X). The JSD head takes the
    teacher's X_teacher [BT, H_t], W_teacher [V, H_t] (+ b_teacher [V]) and no
    ``target``; the ratio heads take ``old_logprobs`` [BT] and the advantages
    as ``weights``.
    """
    _check_head(head, temperature)
    X = _f64(X)
    W = _f64(W)
    BT, H = X.shape
    V = W.shape[0]
    valid = valid_rows(labels, ignore_index, BT)
    n_valid = int(valid.sum())
    g = reduction_scale(head, reduction, n_valid, V)
    L, w, dZ = _rows(head, X, W, b, labels=labels, target=target, weights=weights,
                     valid=valid, g=g, temperature=temperature, eps=eps,
                     X_teacher=X_teacher, W_teacher=W_teacher, b_teacher=b_teacher,
                     old_logprobs=old_logprobs, clip_low=clip_low, clip_high=clip_high)
    loss = g * float((w * L).sum())
    out = dict(loss=loss, per_row=L, n_valid=n_valid, g=g, dW=None, db=None, dZ=dZ)
    out["dX"] = dZ @ W
    if compute_dW:
        out["dW"] = dZ.T @ X
    if compute_db:
        out["db"] = dZ.sum(axis=0)
    return out


def _take(a, rows):
    return None if a is None else a[rows]


def fwd_bwd_blocked(X, W, b=None, *, head, labels=None, target=None, weights=None,
                    reduction="batchmean", ignore_index=-100, temperature=1.0,
                    eps=1e-10, compute_dW=True, compute_db=True, X_teacher=None,
                    W_teacher=None, b_teacher=None, old_logprobs=None, clip_low=0.2,
                    clip_high=0.2, block_rows=512, progress=None):
    """``fwd_bwd`` for shapes whose BT x V logits do not fit in host memory.

    The same arithmetic on blocks of ``block_rows`` token rows: g comes from
    the global valid-row count, each block's per-row terms and dX rows are
    those of ``fwd_bwd`` restricted to the block, dW and db add each block's
    dZ_blk^T X_blk and column sums in row order (a regrouping of the same
    float64 sums), and the loss reduces the whole per-row vector at the end
    exactly as ``fwd_bwd`` does. Inputs may be float32 / bfloat16-valued
    arrays; each block is widened to float64 when it is used. ``progress``
    (optional) is called with (rows done, BT) after every block.
    """
    _check_head(head, temperature)
    W = _f64(W)
    BT, H = X.shape
    V = W.shape[0]
    valid = valid_rows(labels, ignore_index, BT)
    n_valid = int(valid.sum())
    g = reduction_scale(head, reduction, n_valid, V)
    Wt = None if W_teacher is None else _f64(W_teacher)
    L = np.zeros(BT)
    w = np.ones(BT)
    dX = np.zeros((BT, H))
    dW = np.zeros((V, H)) if compute_dW else None
    db = np.zeros(V) if compute_db else None
    for r0 in range(0, BT, block_rows):
        rows = slice(r0, min(BT, r0 + block_rows))
        Xb = _f64(X[rows])
        Lb, wb, dZ = _rows(head, Xb, W, b, labels=_take(labels, rows),
                           target=_take(target, rows), weights=_take(weights, rows),
                           valid=valid[rows], g=g, temperature=temperature, eps=eps,
                           X_teacher=_take(X_teacher, rows), W_teacher=Wt,
                           b_teacher=b_teacher, old_logprobs=_take(old_logprobs, rows),
                           clip_low=clip_low, clip_high=clip_high)
        L[rows] = Lb
        w[rows] = wb
        dX[rows] = dZ @ W
        if compute_dW:
            dW += dZ.T @ Xb
        if compute_db:
            db += dZ.sum(axis=0)
        del dZ, Xb
        if progress is not None:
            progress(rows.stop, BT)
    loss = g * float((w * L).sum())
    return dict(loss=loss, per_row=L, n_valid=n_valid, g=g, dX=dX, dW=dW, db=db)


def sampled_rows(X_rows, W, b=None, *, head, n_valid, labels_rows=None,
                 target_rows=None, weights_rows=None, reduction="batchmean",
                 ignore_index=-100, temperature=1.0, eps=1e-10,
                 Xt_rows=None, W_teacher=None, b_teacher=None, old_logprobs_rows=None,
                 clip_low=0.2, clip_high=0.2):
    """The same definition restricted to a subset of rows.

    Every step above except the final reduction is row-local, so for a subset
    of rows the per-row terms and the dX rows follow from the rows themselves
    and the global valid-row count ``n_valid`` (which fixes g).

    Returns a dict with per_row [R], weighted [R] = g * w_r * L_r (the rows'
    share of the loss) and dX [R, H].
    """
    _check_head(head, temperature)
    X_rows = _f64(X_rows)
    W = _f64(W)
    R = X_rows.shape[0]
    V = W.shape[0]
    valid = valid_rows(labels_rows, ignore_index, R)
    g = reduction_scale(head, reduction, n_valid, V)
    L, w, dZ = _rows(head, X_rows, W, b, labels=labels_rows, target=target_rows,
                     weights=weights_rows, valid=valid, g=g, temperature=temperature,
                     eps=eps, X_teacher=Xt_rows, W_teacher=W_teacher, b_teacher=b_teacher,
                     old_logprobs=old_logprobs_rows, clip_low=clip_low,
                     clip_high=clip_high)
    return dict(per_row=L, weighted=g * w * L, dX=dZ @ W, g=g)
