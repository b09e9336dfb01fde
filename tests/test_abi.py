"""The C-ABI library on the host: symbols, struct layouts, planner, errors.

No GPU is needed: ``fll_plan`` makes no HIP call, and every ``fll_fwd_bwd``
call below carries exactly one defect that the host-side checks reject
before anything is enqueued (the pointers are placeholders and are never
dereferenced).
"""

import ctypes
import os
import re
import subprocess

import pytest

import lm_head_projection_token_amd as fll

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fll.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fll_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    decl = _declared_functions()
    assert "fll_plan" in decl and "fll_fwd_bwd" in decl
    assert set(decl) == set(fll.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fll.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    ver = int(re.search(r"#define FLL_VERSION (\d+)", open(HEADER).read()).group(1))
    assert fll.fll_version() == ver == fll.ABI_VERSION
    out = subprocess.run(["nm", "-D", "--defined-only", fll.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fll_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_struct_layouts_match_the_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(f"""
#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu\\n", sizeof(fll_problem), sizeof(fll_plan_t), sizeof(fll_args),
         sizeof(fll_profile_t));
  printf("%zu\\n", (size_t)FLL_STATIC_SCRATCH_BYTES);
  printf("%zu %zu %zu %zu %zu %zu\\n", offsetof(fll_problem, ignore_index),
         offsetof(fll_plan_t, workspace_bytes), offsetof(fll_args, workspace_bytes),
         offsetof(fll_profile_t, total_ms), offsetof(fll_problem, clip_high),
         offsetof(fll_args, old_logprobs));
  return 0;
}}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-o", str(exe), str(prog)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True,
                           check=True).stdout.split("\n")
    sizes = [int(x) for x in lines[0].split()]
    assert int(lines[1]) == fll.FLL_STATIC_SCRATCH_BYTES
    offs = [int(x) for x in lines[2].split()]
    assert sizes == [ctypes.sizeof(fll.FllProblem), ctypes.sizeof(fll.FllPlan),
                     ctypes.sizeof(fll.FllArgs), ctypes.sizeof(fll.FllProfile)]
    assert offs == [fll.FllProblem.ignore_index.offset, fll.FllPlan.workspace_bytes.offset,
                    fll.FllArgs.workspace_bytes.offset, fll.FllProfile.total_ms.offset,
                    fll.FllProblem.clip_high.offset, fll.FllArgs.old_logprobs.offset]


# --------------------------------------------------------------------------
# planner
# --------------------------------------------------------------------------

def _prob(**kw):
    base = dict(BT=8192, H=4096, V=128256, dtype="bf16", head="selective",
                reduction="mean")
    base.update(kw)
    return fll.make_problem(**base)


@pytest.mark.parametrize("BT,C", [(8192, 4096), (4096, 2048), (1024, 512), (300, 256),
                                  (256, 256), (1, 1), (100000, 8192)])
def test_plan_chunk_policy(BT, C):
    plan = fll.fll_plan(_prob(BT=BT))
    assert plan.chunk_rows == C
    assert plan.n_chunks == -(-BT // C)
    if BT > 256:
        assert plan.n_chunks >= 2  # the BT x V logits are never formed at once
    assert plan.s_pitch >= plan.p.V and plan.s_pitch % 64 == 0
    assert plan.workspace_bytes >= C * plan.s_pitch * 4
    assert plan.workspace_bytes % 256 == 0


def test_plan_does_not_depend_on_gradient_flags():
    a = fll.fll_plan(_prob(compute_dW=False, has_bias=False))
    b = fll.fll_plan(_prob(compute_dW=True, has_bias=True, compute_db=True))
    for f in ("chunk_rows", "n_chunks", "s_pitch", "dx_splits", "dx_split_len",
              "workspace_bytes"):
        assert getattr(a, f) == getattr(b, f), f


def test_plan_dx_split_fills_the_device():
    # the vocabulary split of the dX GEMM targets one workgroup of 256 x 256
    # output tiles per CU (256), keeps >= 2048 vocabulary entries per split,
    # covers V exactly once, and does not depend on the gradient flags
    for BT, V, want in ((8192, 128256, 1), (4096, 128256, 2), (1024, 32000, 8),
                        (300, 1000, 1), (600, 128256, 8), (256, 32000, 15)):
        for flags in (dict(), dict(compute_dW=True, has_bias=True, compute_db=True)):
            pl = fll.fll_plan(_prob(BT=BT, V=V, **flags))
            tiles = -(-pl.chunk_rows // 256) * (4096 // 256)
            assert pl.dx_splits == want, (BT, V, pl.dx_splits)
            assert pl.dx_splits * pl.dx_split_len >= V
            assert (pl.dx_splits - 1) * pl.dx_split_len < V
            assert pl.dx_splits == 1 or V / pl.dx_splits >= 2048 - 64
            assert pl.dx_splits * tiles >= 256 or pl.dx_splits == max(1, min(16, V // 2048))
            assert pl.dx_splits == 1 or (pl.dx_splits - 1) * tiles < 256


def test_plan_budget_shrinks_chunks_then_fails():
    full = fll.fll_plan(_prob())
    small = fll.fll_plan(_prob(), full.workspace_bytes // 3)
    assert small.chunk_rows < full.chunk_rows and small.chunk_rows % 256 == 0
    assert small.workspace_bytes <= full.workspace_bytes // 3
    with pytest.raises(fll.FllError) as e:
        fll.fll_plan(_prob(), 1 << 20)
    assert e.value.status == fll.FLL_ERR_WORKSPACE


def test_plan_forced_chunk_rows():
    plan = fll.fll_plan(_prob(BT=1000), 0, 100)
    assert plan.chunk_rows == 100 and plan.n_chunks == 10
    plan = fll.fll_plan(_prob(BT=50), 0, 100)
    assert plan.chunk_rows == 50 and plan.n_chunks == 1


def test_plan_empty_batch():
    plan = fll.fll_plan(_prob(BT=0))
    assert plan.n_chunks == 0 and plan.workspace_bytes > 0


@pytest.mark.parametrize("kw,status", [
    (dict(reduction="none"), fll.FLL_ERR_UNSUPPORTED),
    (dict(reduction=7), fll.FLL_ERR_INVALID_ARG),
    (dict(temperature=0.0), fll.FLL_ERR_INVALID_ARG),
    (dict(temperature=-1.0), fll.FLL_ERR_INVALID_ARG),
    (dict(temperature=float("nan")), fll.FLL_ERR_INVALID_ARG),
    (dict(temperature=float("inf")), fll.FLL_ERR_INVALID_ARG),
    (dict(eps=-1e-3), fll.FLL_ERR_INVALID_ARG),
    (dict(eps=float("nan")), fll.FLL_ERR_INVALID_ARG),
    (dict(H=4100), fll.FLL_ERR_INVALID_ARG),
    (dict(H=0), fll.FLL_ERR_INVALID_ARG),
    (dict(V=0), fll.FLL_ERR_INVALID_ARG),
    (dict(BT=-1), fll.FLL_ERR_INVALID_ARG),
    (dict(dtype=5), fll.FLL_ERR_INVALID_ARG),
    (dict(head=9), fll.FLL_ERR_INVALID_ARG),
    (dict(compute_db=True, has_bias=False), fll.FLL_ERR_INVALID_ARG),
    (dict(head="jsd"), fll.FLL_ERR_INVALID_ARG),                  # no H_teacher
    (dict(head="jsd", H_teacher=100), fll.FLL_ERR_INVALID_ARG),   # not a multiple of 8
    (dict(head="jsd", H_teacher=4096, teacher_has_bias=2), fll.FLL_ERR_INVALID_ARG),
    (dict(H_teacher=4096), fll.FLL_ERR_INVALID_ARG),              # teacher for another head
    (dict(teacher_has_bias=True), fll.FLL_ERR_INVALID_ARG),
    (dict(logits_bf16=2), fll.FLL_ERR_INVALID_ARG),
    (dict(logits_bf16=True, dtype="fp32"), fll.FLL_ERR_INVALID_ARG),  # bf16 problems only
    (dict(head="ppo", clip_low=-0.1), fll.FLL_ERR_INVALID_ARG),
    (dict(head="ppo", clip_low=1.5), fll.FLL_ERR_INVALID_ARG),
    (dict(head="ppo", clip_low=float("nan")), fll.FLL_ERR_INVALID_ARG),
    (dict(head="cispo", clip_high=-1.0), fll.FLL_ERR_INVALID_ARG),
    (dict(head="cispo", clip_high=float("nan")), fll.FLL_ERR_INVALID_ARG),
    (dict(clip_low=0.2), fll.FLL_ERR_INVALID_ARG),                # clip for another head
    (dict(head="kl", clip_high=0.2), fll.FLL_ERR_INVALID_ARG),
])
def test_plan_rejects(kw, status):
    with pytest.raises(fll.FllError) as e:
        fll.fll_plan(_prob(**kw))
    assert e.value.status == status
    assert fll.fll_last_error()


def test_plan_rejects_negative_chunk_rows():
    with pytest.raises(fll.FllError):
        fll.fll_plan(_prob(), 0, -5)


# --------------------------------------------------------------------------
# fll_fwd_bwd host-side checks (each call has one defect; nothing launches)
# --------------------------------------------------------------------------

A = 1 << 20  # a 256-byte aligned placeholder address, never dereferenced


def _args(plan, **over):
    base = dict(X=A, W=2 * A, b=None, labels=3 * A, target=None, weights=4 * A,
                dX=5 * A, dW=None, db=None, loss=6 * A, per_row=None, workspace=7 * A,
                workspace_bytes=plan.workspace_bytes)
    base.update(over)
    return fll.FllArgs(**base)


def _call(plan, args):
    return fll.lib().fll_fwd_bwd(ctypes.byref(plan), ctypes.byref(args), None)


@pytest.mark.parametrize("over,status", [
    (dict(loss=None), fll.FLL_ERR_INVALID_ARG),
    (dict(loss=6 * A + 2), fll.FLL_ERR_INVALID_ARG),
    (dict(workspace=None), fll.FLL_ERR_WORKSPACE),
    (dict(workspace_bytes=1024), fll.FLL_ERR_WORKSPACE),
    (dict(workspace=7 * A + 64), fll.FLL_ERR_INVALID_ARG),
    (dict(X=None), fll.FLL_ERR_INVALID_ARG),
    (dict(W=None), fll.FLL_ERR_INVALID_ARG),
    (dict(dX=None), fll.FLL_ERR_INVALID_ARG),
    (dict(X=A + 8), fll.FLL_ERR_INVALID_ARG),
    (dict(labels=None), fll.FLL_ERR_INVALID_ARG),
    (dict(labels=3 * A + 4), fll.FLL_ERR_INVALID_ARG),
    (dict(target=8 * A), fll.FLL_ERR_INVALID_ARG),
    (dict(b=9 * A), fll.FLL_ERR_INVALID_ARG),
])
def test_fwd_bwd_rejects_selective(over, status):
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000))
    assert _call(plan, _args(plan, **over)) == status


@pytest.mark.parametrize("over,status", [
    (dict(dW=None), fll.FLL_ERR_INVALID_ARG),
    (dict(dW=10 * A + 4), fll.FLL_ERR_INVALID_ARG),
    (dict(db=None), fll.FLL_ERR_INVALID_ARG),
    (dict(b=None), fll.FLL_ERR_INVALID_ARG),
    (dict(target=None), fll.FLL_ERR_INVALID_ARG),
    (dict(weights=4 * A), fll.FLL_ERR_INVALID_ARG),
])
def test_fwd_bwd_rejects_kl_trainable(over, status):
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000, head="kl", has_bias=True,
                              compute_dW=True, compute_db=True))
    base = dict(labels=None, weights=None, target=8 * A, b=9 * A, dW=10 * A, db=11 * A)
    base.update(over)
    assert _call(plan, _args(plan, **base)) == status


@pytest.mark.parametrize("over,status", [
    (dict(X_teacher=None), fll.FLL_ERR_INVALID_ARG),
    (dict(W_teacher=None), fll.FLL_ERR_INVALID_ARG),
    (dict(X_teacher=12 * A + 8), fll.FLL_ERR_INVALID_ARG),
    (dict(b_teacher=None), fll.FLL_ERR_INVALID_ARG),
    (dict(target=8 * A), fll.FLL_ERR_INVALID_ARG),
    (dict(weights=4 * A), fll.FLL_ERR_INVALID_ARG),
])
def test_fwd_bwd_rejects_jsd(over, status):
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000, head="jsd", H_teacher=96,
                              teacher_has_bias=True))
    base = dict(labels=None, weights=None, X_teacher=12 * A, W_teacher=13 * A,
                b_teacher=14 * A)
    base.update(over)
    assert _call(plan, _args(plan, **base)) == status


def test_plan_accepts_ratio_heads_without_upper_clip():
    for head in ("ppo", "cispo"):
        a = fll.fll_plan(_prob(head=head, clip_low=1.0, clip_high=float("inf")))
        c = fll.fll_plan(_prob(head="selective"))
        assert a.chunk_rows == c.chunk_rows and a.workspace_bytes == c.workspace_bytes


@pytest.mark.parametrize("over,status", [
    (dict(old_logprobs=None), fll.FLL_ERR_INVALID_ARG),
    (dict(old_logprobs=15 * A + 2), fll.FLL_ERR_INVALID_ARG),
    (dict(labels=None), fll.FLL_ERR_INVALID_ARG),
    (dict(target=8 * A), fll.FLL_ERR_INVALID_ARG),
    (dict(X_teacher=12 * A), fll.FLL_ERR_INVALID_ARG),
])
@pytest.mark.parametrize("head", ["ppo", "cispo"])
def test_fwd_bwd_rejects_ratio(over, status, head):
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000, head=head, clip_high=0.28))
    base = dict(old_logprobs=15 * A)
    base.update(over)
    assert _call(plan, _args(plan, **base)) == status


def test_fwd_bwd_rejects_old_logprobs_for_other_heads():
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000))
    assert _call(plan, _args(plan, old_logprobs=15 * A)) == fll.FLL_ERR_INVALID_ARG


def test_fwd_bwd_rejects_teacher_inputs_for_other_heads():
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000))
    assert _call(plan, _args(plan, X_teacher=12 * A)) == fll.FLL_ERR_INVALID_ARG


def test_plan_jsd_adds_the_teacher_chunk():
    # the teacher's logits chunk and statistics come on top of the student's
    a = fll.fll_plan(_prob(head="kl"))
    j = fll.fll_plan(_prob(head="jsd", H_teacher=4096))
    assert j.chunk_rows == a.chunk_rows
    extra = j.workspace_bytes - a.workspace_bytes
    assert extra >= j.chunk_rows * j.s_pitch * 4 + j.chunk_rows * j.stat_tiles * 8
    assert j.off_teacher_stats >= j.off_teacher + j.chunk_rows * j.s_pitch * 4


@pytest.mark.parametrize("head,kw", [("selective", {}), ("kl", {}),
                                     ("jsd", dict(H_teacher=2048))])
def test_plan_bf16_logits_halve_the_chunk(head, kw):
    # bf16 chunk logits: the same chunk size, 2 bytes per logit for the
    # student's (and the teacher's) chunk instead of 4
    f = fll.fll_plan(_prob(head=head, **kw))
    h = fll.fll_plan(_prob(head=head, logits_bf16=True, **kw))
    assert (h.chunk_rows, h.n_chunks, h.s_pitch, h.dx_splits) == \
        (f.chunk_rows, f.n_chunks, f.s_pitch, f.dx_splits)
    n_chunks = 2 if head == "jsd" else 1
    saved = n_chunks * f.chunk_rows * f.s_pitch * 2
    assert f.workspace_bytes - h.workspace_bytes == saved
    assert h.off_rowval - h.off_logits >= h.chunk_rows * h.s_pitch * 2


def test_fwd_bwd_rejects_edited_plan():
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000))
    plan.chunk_rows = 0
    assert _call(plan, _args(plan)) == fll.FLL_ERR_INVALID_ARG
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000))
    plan.dx_splits += 1
    assert _call(plan, _args(plan)) == fll.FLL_ERR_INVALID_ARG
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000))
    plan.p.reduction = fll.FLL_RED_NONE
    assert _call(plan, _args(plan)) == fll.FLL_ERR_UNSUPPORTED


def test_static_entry_point_refusals_before_any_device_call():
    # the scratch-backed call checks its own arguments on the host first
    lib = fll.lib()
    small = fll.fll_plan(_prob(BT=512, H=64, V=1000), fll.FLL_STATIC_SCRATCH_BYTES)
    assert small.workspace_bytes <= fll.FLL_STATIC_SCRATCH_BYTES
    # a caller workspace is refused: the call uses the library's own
    args = _args(small)
    assert lib.fll_fwd_bwd_static(ctypes.byref(small), ctypes.byref(args),
                                  None) == fll.FLL_ERR_INVALID_ARG
    assert "workspace must be NULL" in fll.fll_last_error()
    # a plan made for a larger budget does not fit the scratch
    big = fll.fll_plan(_prob())
    assert big.workspace_bytes > fll.FLL_STATIC_SCRATCH_BYTES
    args = _args(big, workspace=None, workspace_bytes=0)
    assert lib.fll_fwd_bwd_static(ctypes.byref(big), ctypes.byref(args),
                                  None) == fll.FLL_ERR_WORKSPACE
    assert "FLL_STATIC_SCRATCH_BYTES" in fll.fll_last_error()
    assert lib.fll_fwd_bwd_static(None, ctypes.byref(args), None) == fll.FLL_ERR_INVALID_ARG


def test_static_scratch_budget_plans_the_head_shapes():
    # the 512 MiB scratch fits every named head shape at a reduced chunk
    for kw in (dict(), dict(V=151936, has_bias=True, compute_dW=True, compute_db=True),
               dict(head="kl", BT=4096, compute_dW=True),
               dict(head="jsd", BT=4096, H_teacher=4096)):
        plan = fll.fll_plan(_prob(**kw), fll.FLL_STATIC_SCRATCH_BYTES)
        assert plan.workspace_bytes <= fll.FLL_STATIC_SCRATCH_BYTES
        assert plan.chunk_rows >= 256


def test_fwd_bwd_rejects_null_plan_and_args():
    plan = fll.fll_plan(_prob(BT=512, H=64, V=1000))
    assert fll.lib().fll_fwd_bwd(None, ctypes.byref(_args(plan)), None) == \
        fll.FLL_ERR_INVALID_ARG
    assert fll.lib().fll_fwd_bwd(ctypes.byref(plan), None, None) == fll.FLL_ERR_INVALID_ARG


def test_strerror_covers_every_status():
    for s in (0, -1, -2, -3, -4):
        assert fll.fll_strerror(s) and fll.fll_strerror(s) != "unknown status"
    assert fll.fll_strerror(42) == "unknown status"


def test_one_hip_runtime_in_the_process():
    # torch bundles its own HIP runtime; the package must load torch before
    # libfll.so so that both use one runtime (two in one process leave the
    # second without a device).
    code = (
        "import lm_head_projection_token_amd, torch\n"
        "maps = open('/proc/self/maps').read().split('\\n')\n"
        "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
        "print(len(libs)); print(sorted(libs))\n"
    )
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True,
                         cwd=ROOT, check=True).stdout.split("\n")
    assert out[0] == "1", out
