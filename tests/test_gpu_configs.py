"""The five named workloads at full size, in the launch configuration the
benchmark times (the default plan), compared with the oracle element by
element.

cfg1 (tiny fp32) and cfg2 (V = 32000) go through the oracle's materialised
pass. cfg3-cfg5 (and the cross-entropy and Jensen-Shannon heads at the
V = 128256 head shape) go through its row-blocked pass, which has the same
arithmetic and returns the full loss, every per-row term, dX, the whole
[V x H] weight gradient and db: all of them are compared at the stated
tolerances (the fp32 weight-gradient accumulation across chunks,
FusedLinearKLDivLoss page, Details; the fp32 [V, H] gradient of the frozen
lm_head GRPO page, Summary). Each oracle result also serves the same
workload with the chunk logits kept in bf16.
"""

import numpy as np
import pytest
import torch

import workloads
from tests import helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_cfg1_full():
    case = workloads.WORKLOADS[1]
    inp = H.make(case)
    H.compare_full(H.run_gpu(inp, case), H.run_oracle(inp, case), case)


def test_cfg2_full():
    case = workloads.WORKLOADS[2]
    print(f"[cfg2] {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    ref = H.run_oracle(inp, case)
    H.compare_full(out, ref, case)


# The fused linear cross-entropy head at the llama-3 head shape of the
# V=128256 GRPO workload, with a trainable head (beyond the five workloads).
CE_FULL = workloads.WORKLOADS[3].replace(name="ce-bf16-trainable-B8T1024-V128256", head="ce",
                                         compute_dW=True, ignore_frac=0.05, seed=6)
# The PPO clipped surrogate (the GRPO family) at the same shape, with a
# trainable head and ignored rows; its old log-probs are the oracle's
# log p(y) minus drawn log-ratios kept off the clip edges.
PPO_FULL = workloads.PPO_WORKLOAD.replace(name="ppo-bf16-trainable-B8T1024-V128256",
                                          compute_dW=True, ignore_frac=0.05)
EXTRA = {"ce": CE_FULL, "jsd": workloads.JSD_WORKLOAD, "ppo": PPO_FULL}

# which workloads are also run with bf16 chunk logits against the same oracle
BF16_LOGITS_TOO = {3, 5, "jsd"}


def _compare(out, ref, case, inp, logits_bf16):
    H.check_loss(float(out["loss"]), ref["loss"], case.dtype)
    per = H.to_np(out["per_row"])
    scale = float(np.abs(ref["per_row"]).max())
    atol = 2e-3 * scale
    # plus what rounding the logits to bf16 can move a row's term; the label
    # heads take the label's logit in fp32 from the GEMM, so theirs do not move
    if logits_bf16 and case.head not in workloads.LABEL_HEADS:
        atol = atol + H.logit_rounding_bound(inp, case)
    err = np.abs(per - ref["per_row"])
    bad = err > atol + 2e-3 * np.abs(ref["per_row"])
    assert not bad.any(), f"per_row: {int(bad.sum())} rows out, max err {err.max():.3e}"
    H.check_grad(out["dX"].float().cpu().numpy(), ref["dX"], case.dtype, "dX")
    if case.compute_dW:
        H.check_grad(out["dW"].cpu().numpy(), ref["dW"], case.dtype, "dW")
    if case.compute_db:
        H.check_grad(out["db"].cpu().numpy(), ref["db"], case.dtype, "db")
    labels = inp["labels"]
    if labels is not None:
        ign = (labels == case.ignore_index)
        if bool(ign.any()):
            assert torch.count_nonzero(out["dX"].cpu()[ign]).item() == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [3, 4, 5, "ce", "jsd", "ppo"])
def test_full_config(cfg):
    case = EXTRA[cfg] if cfg in EXTRA else workloads.WORKLOADS[cfg]
    print(f"[cfg{cfg}] {case}", flush=True)
    inp = H.make(case)
    out = H.run_gpu(inp, case)
    print(f"[cfg{cfg}] GPU done; oracle (row-blocked, full size)", flush=True)
    ref = H.run_oracle_blocked(inp, case, tag=f"cfg{cfg}")
    print(f"[cfg{cfg}] oracle done; comparing", flush=True)
    _compare(out, ref, case, inp, logits_bf16=False)
    del out
    if cfg in BF16_LOGITS_TOO:
        print(f"[cfg{cfg}] bf16 chunk logits", flush=True)
        out = H.run_gpu(inp, case, logits_bf16=True)
        _compare(out, ref, case, inp, logits_bf16=True)
    print(f"[cfg{cfg}] ok", flush=True)
