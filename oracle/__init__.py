"""CPU float64 oracle (test infrastructure only; see ``fll_oracle``)."""

from .fll_oracle import (  # noqa: F401
    HEAD_CE,
    HEAD_JSD,
    HEAD_KL,
    HEAD_SELECTIVE,
    ce_rows,
    dlogits,
    fwd_bwd,
    jsd_rows,
    kl_rows,
    log_softmax,
    logits,
    reduction_scale,
    row_weights,
    sampled_rows,
    selective_rows,
    teacher_probs,
    valid_rows,
)
