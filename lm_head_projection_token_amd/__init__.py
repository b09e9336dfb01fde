"""Python binding of ``libfll.so``: the fused lm_head loss for MI355X.

This module only marshals arguments into the C ABI declared in
``include/fll.h``: every step of the computation runs in the library's HIP
kernels. PyTorch is used for device memory and the current stream.

The names mirror the C entry points: ``fll_plan``, ``fll_fwd_bwd``,
``fll_strerror``, ``fll_last_error``, ``fll_version``,
``fll_profile_enable`` and ``fll_profile_read``. ``fused_lm_head_loss`` is a
convenience wrapper that allocates the outputs and the workspace with torch
and calls ``fll_plan`` + ``fll_fwd_bwd``.

The library must be built (``python lm_head_projection_token_amd/build.py``);
importing this package without it raises, there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# FLL_LIBRARY names another build of the same library (the host-sanitized
# one the CPU tests build); by default the in-tree libfll.so
LIB_PATH = os.environ.get("FLL_LIBRARY") or os.path.join(PKG, "libfll.so")
ABI_VERSION = 4  # FLL_VERSION of include/fll.h that the structs below mirror

FLL_OK = 0
FLL_ERR_INVALID_ARG = -1
FLL_ERR_UNSUPPORTED = -2
FLL_ERR_WORKSPACE = -3
FLL_ERR_HIP = -4

FLL_HEAD_KL = 0
FLL_HEAD_SELECTIVE_LOGPROB = 1
FLL_HEAD_CROSS_ENTROPY = 2
FLL_HEAD_JSD = 3
FLL_HEAD_PPO_CLIP = 4
FLL_HEAD_CISPO = 5
HEADS = {"kl": FLL_HEAD_KL, "selective": FLL_HEAD_SELECTIVE_LOGPROB,
         "ce": FLL_HEAD_CROSS_ENTROPY, "jsd": FLL_HEAD_JSD, "ppo": FLL_HEAD_PPO_CLIP,
         "cispo": FLL_HEAD_CISPO}
RATIO_HEADS = ("ppo", "cispo", FLL_HEAD_PPO_CLIP, FLL_HEAD_CISPO)

FLL_RED_BATCHMEAN, FLL_RED_MEAN, FLL_RED_SUM, FLL_RED_NONE = 0, 1, 2, 3
REDUCTIONS = {"batchmean": 0, "mean": 1, "sum": 2, "none": 3}

FLL_BF16, FLL_FP32 = 0, 1
DTYPES = {"bf16": FLL_BF16, "fp32": FLL_FP32}

KERNEL_KINDS = ["prep", "logits", "row", "dx", "dx_reduce", "dw", "db", "final",
                "teacher", "transpose"]


class FllProblem(ctypes.Structure):
    _fields_ = [
        ("BT", ctypes.c_int64), ("H", ctypes.c_int64), ("V", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("head", ctypes.c_int32),
        ("has_bias", ctypes.c_int32), ("compute_dW", ctypes.c_int32),
        ("compute_db", ctypes.c_int32), ("reduction", ctypes.c_int32),
        ("ignore_index", ctypes.c_int64), ("temperature", ctypes.c_float),
        ("eps", ctypes.c_float), ("H_teacher", ctypes.c_int64),
        ("teacher_has_bias", ctypes.c_int32), ("logits_bf16", ctypes.c_int32),
        ("clip_low", ctypes.c_float), ("clip_high", ctypes.c_float),
    ]


class FllPlan(ctypes.Structure):
    _fields_ = [
        ("p", FllProblem), ("chunk_rows", ctypes.c_int64),
        ("n_chunks", ctypes.c_int64), ("s_pitch", ctypes.c_int64),
        ("dx_splits", ctypes.c_int64), ("dx_split_len", ctypes.c_int64),
        ("stat_tiles", ctypes.c_int64), ("off_logits", ctypes.c_size_t),
        ("off_rowval", ctypes.c_size_t), ("off_stats", ctypes.c_size_t),
        ("off_dx_partial", ctypes.c_size_t), ("off_scalars", ctypes.c_size_t),
        ("off_teacher", ctypes.c_size_t), ("off_teacher_stats", ctypes.c_size_t),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class FllArgs(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p), ("W", ctypes.c_void_p), ("b", ctypes.c_void_p),
        ("labels", ctypes.c_void_p), ("target", ctypes.c_void_p),
        ("weights", ctypes.c_void_p), ("dX", ctypes.c_void_p),
        ("dW", ctypes.c_void_p), ("db", ctypes.c_void_p),
        ("loss", ctypes.c_void_p), ("per_row", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("X_teacher", ctypes.c_void_p), ("W_teacher", ctypes.c_void_p),
        ("b_teacher", ctypes.c_void_p), ("old_logprobs", ctypes.c_void_p),
    ]


class FllProfile(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * len(KERNEL_KINDS)),
                ("total_ms", ctypes.c_double * len(KERNEL_KINDS))]


class FllError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{fll_strerror(status)} ({status}): {detail}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python lm_head_projection_token_amd/build.py`")
    # torch ships its own HIP and HSA runtimes. Loading torch first lets
    # libfll.so's libamdhip64.so.7 dependency resolve to torch's copy (same
    # soname), so the process holds one runtime; loaded the other way round,
    # two runtimes end up in one process and the second sees no device.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    lib.fll_plan.argtypes = [ctypes.POINTER(FllProblem), ctypes.c_size_t, ctypes.c_int64,
                             ctypes.POINTER(FllPlan)]
    lib.fll_plan.restype = ctypes.c_int
    lib.fll_fwd_bwd.argtypes = [ctypes.POINTER(FllPlan), ctypes.POINTER(FllArgs),
                                ctypes.c_void_p]
    lib.fll_fwd_bwd.restype = ctypes.c_int
    lib.fll_fwd_bwd_static.argtypes = [ctypes.POINTER(FllPlan), ctypes.POINTER(FllArgs),
                                       ctypes.c_void_p]
    lib.fll_fwd_bwd_static.restype = ctypes.c_int
    lib.fll_strerror.argtypes = [ctypes.c_int]
    lib.fll_strerror.restype = ctypes.c_char_p
    lib.fll_last_error.argtypes = []
    lib.fll_last_error.restype = ctypes.c_char_p
    lib.fll_version.argtypes = []
    lib.fll_version.restype = ctypes.c_int
    lib.fll_profile_enable.argtypes = [ctypes.c_int]
    lib.fll_profile_enable.restype = ctypes.c_int
    lib.fll_profile_read.argtypes = [ctypes.POINTER(FllProfile), ctypes.c_int]
    lib.fll_profile_read.restype = ctypes.c_int
    if lib.fll_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.fll_version()}, this binding "
                          f"needs {ABI_VERSION}: rebuild it")
    return lib


_lib = _load()

# Symbols declared in include/fll.h (checked by the CPU tests).
EXPORTS = ("fll_plan", "fll_fwd_bwd", "fll_fwd_bwd_static", "fll_strerror",
           "fll_last_error", "fll_version", "fll_profile_enable", "fll_profile_read")

# bytes of the library's per-device scratch used by fll_fwd_bwd_static
FLL_STATIC_SCRATCH_BYTES = 512 << 20


def lib():
    return _lib


def fll_strerror(status: int) -> str:
    return _lib.fll_strerror(status).decode()


def fll_last_error() -> str:
    return _lib.fll_last_error().decode()


def fll_version() -> int:
    return _lib.fll_version()


def _check(status: int):
    if status != FLL_OK:
        raise FllError(status, fll_last_error())


def make_problem(BT, H, V, *, dtype="bf16", head="kl", has_bias=False, compute_dW=False,
                 compute_db=False, reduction="batchmean", ignore_index=-100,
                 temperature=1.0, eps=1e-10, H_teacher=0,
                 teacher_has_bias=False, logits_bf16=False, clip_low=None,
                 clip_high=None) -> FllProblem:
    """The ratio heads' clip widths default to 0.2 each; other heads take 0."""
    ratio = head in RATIO_HEADS
    if clip_low is None:
        clip_low = 0.2 if ratio else 0.0
    if clip_high is None:
        clip_high = 0.2 if ratio else 0.0
    return FllProblem(
        BT=BT, H=H, V=V, dtype=DTYPES[dtype] if isinstance(dtype, str) else dtype,
        head=HEADS[head] if isinstance(head, str) else head,
        has_bias=int(has_bias), compute_dW=int(compute_dW), compute_db=int(compute_db),
        reduction=REDUCTIONS[reduction] if isinstance(reduction, str) else reduction,
        ignore_index=ignore_index, temperature=temperature, eps=eps, H_teacher=H_teacher,
        teacher_has_bias=int(teacher_has_bias), logits_bf16=int(logits_bf16),
        clip_low=clip_low, clip_high=clip_high)


def fll_plan(problem: FllProblem, max_workspace_bytes: int = 0,
             chunk_rows: int = 0) -> FllPlan:
    """Plan a problem (host only). Raises FllError on a bad problem."""
    plan = FllPlan()
    _check(_lib.fll_plan(ctypes.byref(problem), max_workspace_bytes, chunk_rows,
                         ctypes.byref(plan)))
    return plan


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def fll_fwd_bwd(plan: FllPlan, *, X, W, b=None, labels=None, target=None, weights=None,
                dX, dW=None, db=None, loss, per_row=None, workspace,
                workspace_bytes: Optional[int] = None, stream=None, X_teacher=None,
                W_teacher=None, b_teacher=None, old_logprobs=None) -> None:
    """Enqueue one fused forward + backward on ``stream`` (torch stream,
    raw handle int, or None for torch's current stream). Tensors must be
    contiguous device tensors of the dtypes ``include/fll.h`` states."""
    import torch

    for name, t in (("X", X), ("W", W), ("b", b), ("labels", labels), ("target", target),
                    ("weights", weights), ("dX", dX), ("dW", dW), ("db", db),
                    ("loss", loss), ("per_row", per_row), ("workspace", workspace),
                    ("X_teacher", X_teacher), ("W_teacher", W_teacher),
                    ("b_teacher", b_teacher), ("old_logprobs", old_logprobs)):
        if isinstance(t, torch.Tensor) and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if isinstance(
            workspace, torch.Tensor) else plan.workspace_bytes
    args = FllArgs(X=_ptr(X), W=_ptr(W), b=_ptr(b), labels=_ptr(labels),
                   target=_ptr(target), weights=_ptr(weights), dX=_ptr(dX), dW=_ptr(dW),
                   db=_ptr(db), loss=_ptr(loss), per_row=_ptr(per_row),
                   workspace=_ptr(workspace), workspace_bytes=workspace_bytes,
                   X_teacher=_ptr(X_teacher), W_teacher=_ptr(W_teacher),
                   b_teacher=_ptr(b_teacher), old_logprobs=_ptr(old_logprobs))
    if stream is None:
        handle = torch.cuda.current_stream().cuda_stream
    elif isinstance(stream, int):
        handle = stream
    else:
        handle = stream.cuda_stream
    _check(_lib.fll_fwd_bwd(ctypes.byref(plan), ctypes.byref(args), ctypes.c_void_p(handle)))


def fll_fwd_bwd_static(plan: FllPlan, *, X, W, b=None, labels=None, target=None,
                       weights=None, dX, dW=None, db=None, loss, per_row=None, stream=None,
                       X_teacher=None, W_teacher=None, b_teacher=None,
                       old_logprobs=None) -> None:
    """``fll_fwd_bwd`` with the library's static per-device scratch as the
    workspace (plan with ``max_workspace_bytes=FLL_STATIC_SCRATCH_BYTES``):
    allocates nothing. Calls that overlap on one device race."""
    import torch

    for name, t in (("X", X), ("W", W), ("b", b), ("labels", labels), ("target", target),
                    ("weights", weights), ("dX", dX), ("dW", dW), ("db", db),
                    ("loss", loss), ("per_row", per_row), ("X_teacher", X_teacher),
                    ("W_teacher", W_teacher), ("b_teacher", b_teacher),
                    ("old_logprobs", old_logprobs)):
        if isinstance(t, torch.Tensor) and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    args = FllArgs(X=_ptr(X), W=_ptr(W), b=_ptr(b), labels=_ptr(labels),
                   target=_ptr(target), weights=_ptr(weights), dX=_ptr(dX), dW=_ptr(dW),
                   db=_ptr(db), loss=_ptr(loss), per_row=_ptr(per_row), workspace=None,
                   workspace_bytes=0, X_teacher=_ptr(X_teacher), W_teacher=_ptr(W_teacher),
                   b_teacher=_ptr(b_teacher), old_logprobs=_ptr(old_logprobs))
    if stream is None:
        handle = torch.cuda.current_stream().cuda_stream
    elif isinstance(stream, int):
        handle = stream
    else:
        handle = stream.cuda_stream
    _check(_lib.fll_fwd_bwd_static(ctypes.byref(plan), ctypes.byref(args),
                                   ctypes.c_void_p(handle)))


def fll_profile_enable(enable: bool = True) -> None:
    _check(_lib.fll_profile_enable(int(enable)))


def fll_profile_read(reset: bool = False) -> dict:
    prof = FllProfile()
    _check(_lib.fll_profile_read(ctypes.byref(prof), int(reset)))
    return {k: (prof.launches[i], prof.total_ms[i]) for i, k in enumerate(KERNEL_KINDS)}


def fused_lm_head_loss(X, W, b=None, *, head, labels=None, target=None, weights=None,
                       reduction="batchmean", ignore_index=-100, temperature=1.0, eps=1e-10,
                       compute_dW=False, compute_db=False, chunk_rows=0, per_row=False,
                       workspace=None, X_teacher=None, W_teacher=None, b_teacher=None,
                       logits_bf16=False, old_logprobs=None, clip_low=None,
                       clip_high=None):
    """Allocate outputs with torch and run the fused loss. Returns a dict with
    loss (0-dim fp32 tensor), dX, dW, db and (if asked) per_row. The JSD head
    takes the teacher's X_teacher [BT, H_t], W_teacher [V, H_t] (+ b_teacher);
    the ratio heads ("ppo", "cispo") take old_logprobs [BT] fp32, the
    advantages as weights and the clip widths. logits_bf16 keeps the chunk
    logits in bf16 (bf16 inputs only)."""
    import torch

    dev = X.device
    BT, H = X.shape
    V = W.shape[0]
    dtype = {torch.bfloat16: "bf16", torch.float32: "fp32"}[X.dtype]
    H_t = X_teacher.shape[1] if X_teacher is not None else 0
    prob = make_problem(BT, H, V, dtype=dtype, head=head, has_bias=b is not None,
                        compute_dW=compute_dW, compute_db=compute_db, reduction=reduction,
                        ignore_index=ignore_index, temperature=temperature, eps=eps,
                        H_teacher=H_t, teacher_has_bias=b_teacher is not None,
                        logits_bf16=logits_bf16, clip_low=clip_low, clip_high=clip_high)
    plan = fll_plan(prob, 0, chunk_rows)
    if workspace is None or workspace.numel() < plan.workspace_bytes:
        workspace = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device=dev)
    out = dict(
        loss=torch.empty((), dtype=torch.float32, device=dev),
        dX=torch.empty_like(X),
        dW=torch.empty(V, H, dtype=torch.float32, device=dev) if compute_dW else None,
        db=torch.empty(V, dtype=torch.float32, device=dev) if compute_db else None,
        per_row=torch.empty(BT, dtype=torch.float32, device=dev) if per_row else None,
    )
    fll_fwd_bwd(plan, X=X, W=W, b=b, labels=labels, target=target, weights=weights,
                dX=out["dX"], dW=out["dW"], db=out["db"], loss=out["loss"],
                per_row=out["per_row"], workspace=workspace, X_teacher=X_teacher,
                W_teacher=W_teacher, b_teacher=b_teacher, old_logprobs=old_logprobs)
    out["plan"] = plan
    return out
