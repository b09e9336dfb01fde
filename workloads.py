"""Seeded synthetic inputs for the fused lm_head loss.

This module only draws random inputs. It holds none of the loss arithmetic,
so both the CPU oracle (``oracle/``) and the HIP path (through
``lm_head_projection_token_amd``) can consume the very same tensors.

The five named workloads follow the head shapes the pages measure: a
llama-3 style head (H=4096, V=128256) [FusedLinearKLDivLoss page, Details],
a Qwen-style V=151936 head and B=8, T=1024 GRPO batches [frozen lm_head
GRPO page, Details], plus a tiny fp32 case and a V=32000 distillation case.
Every tensor is drawn in float32 from ``torch.Generator('cpu')`` seeded per
case, in a fixed order (X, W, b, target logits, labels, advantages, ignore
permutation), then cast to bfloat16 with round-to-nearest-even where the
case is bf16. "N(0, s)" means a normal with standard deviation s.

The target distribution of a KL case is the softmax of N(0, s_t) logits in
float32: it is an *input* of the method (an explicit teacher distribution),
so preparing it here is input generation, not the loss arithmetic. Rows
marked ``ignore_index`` get NaN targets so that any read of them shows up.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

HEAD_KL = "kl"
HEAD_SELECTIVE = "selective"
HEAD_CE = "ce"
HEAD_JSD = "jsd"
HEAD_PPO = "ppo"
HEAD_CISPO = "cispo"
LABEL_HEADS = (HEAD_SELECTIVE, HEAD_CE, HEAD_PPO, HEAD_CISPO)
RATIO_HEADS = (HEAD_PPO, HEAD_CISPO)

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Case:
    """A fully specified synthetic workload."""

    name: str
    BT: int
    H: int
    V: int
    dtype: str  # "bf16" or "fp32"
    head: str  # HEAD_KL, HEAD_SELECTIVE, HEAD_CE, HEAD_JSD, HEAD_PPO or HEAD_CISPO
    has_bias: bool = False
    compute_dW: bool = False
    compute_db: bool = False
    reduction: str = "batchmean"
    temperature: float = 1.0
    ignore_frac: float = 0.0
    with_labels: bool = True  # KL: labels act only as an ignore mask
    with_weights: bool = True  # selective and ratio heads: per-token advantages (never CE)
    x_std: float = 1.0
    w_std: float = 0.02
    b_std: float = 0.01
    target_std: float = 2.0
    eps: float = 1e-10
    ignore_index: int = IGNORE_INDEX
    seed: int = 0
    # JSD head: the teacher's own projection X_t [BT, H_teacher] W_t^T (+ b_t)
    H_teacher: int = 0
    teacher_has_bias: bool = False
    teacher_w_std: float = 0.02
    # ratio heads: clip widths of the ratio rho and the spread of the drawn
    # log-ratios log rho (the old log-probs are formed from them by the tests)
    clip_low: float = 0.2
    clip_high: float = 0.2
    logratio_std: float = 0.3

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


# The five workloads. Seeds are the case numbers.
WORKLOADS = {
    1: Case("tiny-fp32-kl-trainable-bias", BT=64, H=256, V=1024, dtype="fp32",
            head=HEAD_KL, has_bias=True, compute_dW=True, compute_db=True,
            reduction="batchmean", x_std=0.02, w_std=0.02, b_std=0.01,
            target_std=1.0, with_labels=False, seed=1),
    2: Case("kl-distill-bf16-frozen-V32000", BT=1024, H=4096, V=32000,
            dtype="bf16", head=HEAD_KL, reduction="batchmean",
            target_std=2.0, with_labels=False, seed=2),
    3: Case("grpo-bf16-frozen-B8T1024-V128256", BT=8192, H=4096, V=128256,
            dtype="bf16", head=HEAD_SELECTIVE, reduction="mean", seed=3),
    4: Case("grpo-bf16-trainable-bias-B8T1024-V151936", BT=8192, H=4096,
            V=151936, dtype="bf16", head=HEAD_SELECTIVE, has_bias=True,
            compute_dW=True, compute_db=True, reduction="mean", seed=4),
    5: Case("kl-distill-bf16-trainable-tau2-V128256", BT=4096, H=4096,
            V=128256, dtype="bf16", head=HEAD_KL, compute_dW=True,
            reduction="batchmean", temperature=2.0, ignore_frac=0.1,
            target_std=2.0, seed=5),
}


# The Jensen-Shannon head at the llama-3 head shape: a student and a teacher
# projection of the same hidden size over V = 128256, frozen student head,
# 4096 tokens (the distillation batch of the KL workload above).
JSD_WORKLOAD = Case("jsd-distill-bf16-frozen-V128256", BT=4096, H=4096, V=128256,
                    dtype="bf16", head=HEAD_JSD, reduction="batchmean", H_teacher=4096,
                    ignore_frac=0.1, seed=9)


# The PPO clipped surrogate (DAPO's wider upper clip) on the frozen GRPO
# workload's shape: B=8, T=1024, H=4096, V=128256, advantages ~ N(0, 1).
PPO_WORKLOAD = Case("ppo-bf16-frozen-B8T1024-V128256", BT=8192, H=4096, V=128256,
                    dtype="bf16", head=HEAD_PPO, reduction="mean", clip_low=0.2,
                    clip_high=0.28, seed=7)


def _normal(gen: torch.Generator, shape, std: float) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.float32)
    t.normal_(0.0, std, generator=gen)
    return t


def make_inputs(case: Case) -> dict:
    """Draw every input of ``case`` on the CPU.

    Returns a dict of CPU tensors: ``X [BT,H]``, ``W [V,H]``, ``b [V]`` or
    None (same dtype as X), ``target [BT,V]`` float32 or None, ``labels
    [BT]`` int64 or None, ``weights [BT]`` float32 or None, the JSD
    teacher's ``X_teacher [BT,H_t]``, ``W_teacher [V,H_t]``, ``b_teacher
    [V]`` (else None), the ratio heads' drawn log-ratios ``logratio [BT]``
    float32 (else None), plus ``case``. The ratio heads' old log-probs depend
    on the model's own log-probs, so the tests form them (old = log p(y) -
    logratio, with log p(y) from the oracle); they are not drawn here.
    """
    gen = torch.Generator("cpu")
    gen.manual_seed(case.seed)
    dt = case.torch_dtype
    BT, H, V = case.BT, case.H, case.V

    X = _normal(gen, (BT, H), case.x_std).to(dt)
    W = _normal(gen, (V, H), case.w_std).to(dt)
    b = _normal(gen, (V,), case.b_std).to(dt) if case.has_bias else None

    target = None
    if case.head == HEAD_KL:
        tl = _normal(gen, (BT, V), case.target_std)
        target = torch.softmax(tl, dim=-1)
        del tl

    labels = None
    need_labels = (case.head in LABEL_HEADS or case.with_labels
                   or case.ignore_frac > 0)
    if need_labels:
        labels = torch.randint(0, V, (BT,), generator=gen, dtype=torch.int64)

    weights = None
    if case.head in (HEAD_SELECTIVE,) + RATIO_HEADS and case.with_weights:
        weights = _normal(gen, (BT,), 1.0)

    if case.ignore_frac > 0 and BT > 0:
        n_ign = int(round(case.ignore_frac * BT))
        perm = torch.randperm(BT, generator=gen)
        ign = perm[:n_ign]
        labels[ign] = case.ignore_index
        if target is not None:
            target[ign] = float("nan")

    # the JSD teacher is drawn last, so the other heads' streams are unchanged
    X_t = W_t = b_t = None
    if case.head == HEAD_JSD:
        X_t = _normal(gen, (BT, case.H_teacher), case.x_std).to(dt)
        W_t = _normal(gen, (V, case.H_teacher), case.teacher_w_std).to(dt)
        if case.teacher_has_bias:
            b_t = _normal(gen, (V,), case.b_std).to(dt)

    # the ratio heads' per-token log-ratios log(pi / pi_old), drawn last
    logratio = None
    if case.head in RATIO_HEADS:
        logratio = _normal(gen, (BT,), case.logratio_std)

    return dict(X=X, W=W, b=b, target=target, labels=labels, weights=weights,
                X_teacher=X_t, W_teacher=W_t, b_teacher=b_t, logratio=logratio,
                case=case)


def small_case(BT=300, H=264, V=1000, *, dtype="bf16", head=HEAD_KL, seed=100,
               **kw) -> Case:
    """A case sized for a full element-wise oracle comparison."""
    return Case(name=f"small-{head}-{dtype}-{BT}x{H}x{V}", BT=BT, H=H, V=V,
                dtype=dtype, head=head, seed=seed, **kw)


def row_sample(BT: int, n: int, seed: int = 1234, labels: Optional[torch.Tensor] = None,
               ignore_index: int = IGNORE_INDEX) -> torch.Tensor:
    """Seeded sorted row indices for sampled full-size checks.

    Always includes the first and last row; if ``labels`` is given, includes
    one ignored row when there is one.
    """
    gen = torch.Generator("cpu")
    gen.manual_seed(seed)
    idx = set(torch.randperm(BT, generator=gen)[: max(0, n - 3)].tolist())
    idx.update({0, BT - 1})
    if labels is not None:
        ign = (labels == ignore_index).nonzero().flatten()
        if ign.numel():
            idx.add(int(ign[0]))
    return torch.tensor(sorted(idx), dtype=torch.int64)
