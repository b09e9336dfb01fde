"""Write the golden regression fixtures from the CPU oracle.

Run from the repository root: ``python tests/golden/make_golden.py``. It
calls only ``oracle/`` (on inputs from ``workloads``) and stores the results
as text, so that a later change to the oracle's arithmetic shows up as a
failing ``test_golden.py`` and has to be justified.
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads  # noqa: E402
from oracle import fll_oracle  # noqa: E402
from tests import helpers  # noqa: E402

CASES = {
    # KL distillation, bf16 inputs, trainable head with bias, ignored rows.
    "kl_bf16_small": workloads.small_case(
        BT=12, H=16, V=40, dtype="bf16", head="kl", has_bias=True,
        compute_dW=True, compute_db=True, temperature=2.0, ignore_frac=0.25,
        seed=7),
    # Selective log-prob, fp32 inputs, frozen head.
    "selective_fp32_small": workloads.small_case(
        BT=10, H=8, V=33, dtype="fp32", head="selective", reduction="mean",
        x_std=1.0, w_std=0.5, seed=8),
    # Jensen-Shannon head, bf16 inputs, teacher of another hidden size with a
    # bias, trainable student head, ignored rows.
    "jsd_bf16_small": workloads.small_case(
        BT=12, H=16, V=40, dtype="bf16", head="jsd", has_bias=True, compute_dW=True,
        compute_db=True, H_teacher=24, teacher_has_bias=True, teacher_w_std=0.3,
        temperature=2.0, ignore_frac=0.25, w_std=0.3, seed=10),
    # PPO clipped surrogate with DAPO's wider upper clip, bf16 inputs,
    # trainable head with bias, ignored rows; old log-probs = the oracle's
    # log p(y) minus drawn log-ratios of spread 0.4 (both clip branches).
    "ppo_bf16_small": workloads.small_case(
        BT=14, H=16, V=40, dtype="bf16", head="ppo", has_bias=True, compute_dW=True,
        compute_db=True, clip_low=0.2, clip_high=0.28, logratio_std=0.4,
        temperature=2.0, ignore_frac=0.2, w_std=0.3, reduction="mean", seed=25),
    # CISPO, fp32 inputs, frozen head, sum reduction.
    "cispo_fp32_small": workloads.small_case(
        BT=10, H=8, V=33, dtype="fp32", head="cispo", clip_low=0.2, clip_high=0.28,
        logratio_std=0.4, reduction="sum", x_std=1.0, w_std=0.5, seed=26),
}


def run_case(case):
    inp = workloads.make_inputs(case)

    def np_(t):
        return None if t is None else t.double().numpy()

    out = fll_oracle.fwd_bwd(
        np_(inp["X"]), np_(inp["W"]), np_(inp["b"]), head=case.head,
        labels=None if inp["labels"] is None else inp["labels"].numpy(),
        target=np_(inp["target"]), weights=np_(inp["weights"]),
        reduction=case.reduction, ignore_index=case.ignore_index,
        temperature=case.temperature, eps=case.eps,
        compute_dW=case.compute_dW, compute_db=case.compute_db,
        X_teacher=np_(inp["X_teacher"]), W_teacher=np_(inp["W_teacher"]),
        b_teacher=np_(inp["b_teacher"]), **helpers._ratio_kw(inp, case))
    rec = dict(loss=out["loss"], per_row=out["per_row"].tolist(),
               n_valid=out["n_valid"], dX_row0=out["dX"][0].tolist(),
               dX_sum=float(out["dX"].sum()))
    if out["dW"] is not None:
        rec["dW_row0"] = out["dW"][0].tolist()
    if out["db"] is not None:
        rec["db"] = out["db"].tolist()
    return rec


def main():
    for name, case in CASES.items():
        path = os.path.join(HERE, f"{name}.json")
        with open(path, "w") as f:
            json.dump(dict(case=case.name, source="oracle/fll_oracle.py fwd_bwd",
                           values=run_case(case)), f, indent=1)
        print("wrote", path)


if __name__ == "__main__":
    main()
