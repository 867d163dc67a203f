"""ctypes binding of liblce.so (include/lce.h), with torch for memory and streams.

Argument marshalling only: every step of the computation runs in the HIP
library.  The functions named ``lce_*`` mirror the C entry points one to one
and take torch tensors already resident on the GPU; ``forward`` and
``backward`` allocate the outputs and the workspace with torch and call them
on the current stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblce.so")

LCE_F32, LCE_BF16 = 0, 1
LCE_MEAN, LCE_SUM = 0, 1
_REDUCTIONS = {"mean": LCE_MEAN, "sum": LCE_SUM}
_DTYPES = {torch.float32: LCE_F32, torch.bfloat16: LCE_BF16}


class LceError(RuntimeError):
    """A call into liblce.so returned a non-OK status."""


class Problem(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("vocab", ctypes.c_int64), ("strip", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reduction", ctypes.c_int32),
                ("ignore_index", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.POINTER(Problem)
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "lce_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lce_pick_strip": (_I64, [_P, _SZ]),
    "lce_workspace_bytes": (_SZ, [_P]),
    "lce_forward_fold_max": (_I64, [_P]),
    "lce_backward_fold_gemm_launches": (ctypes.c_int, [_P, _I64]),
    "lce_backward_fused_workspace_bytes": (_SZ, [_P, ctypes.c_int]),
    "lce_backward_fused": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int,
                                          _VP, _SZ, _VP]),
    "lce_forward": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lce_backward": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lce_forward_begin": (ctypes.c_int, [_P, _VP, _SZ, _VP]),
    "lce_forward_fold": (ctypes.c_int, [_P, _VP, _VP, _I64, _I64, _VP, _VP, _SZ, _VP]),
    "lce_forward_end": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "lce_forward_state": (ctypes.c_int, [_P, _VP, _VP, _SZ, _VP]),
    "lce_forward_merge_state": (ctypes.c_int, [_P, _VP, _VP, _SZ, _VP]),
    "lce_backward_begin": (ctypes.c_int, [_P, _VP, _VP, _VP, _SZ, _VP]),
    "lce_backward_static": (ctypes.c_int, [_P, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "lce_backward_fold": (ctypes.c_int, [_P, _VP, _VP, _I64, _I64, _VP, _VP, _VP, ctypes.c_int,
                                         _VP, _VP, _SZ, _VP]),
    "lce_forward_fold_steps": (ctypes.c_int, [_P, _VP, _VP, _I64, _I64, _VP, _VP, _SZ,
                                              ctypes.c_uint, _VP]),
    "lce_backward_fold_steps": (ctypes.c_int, [_P, _VP, _VP, _I64, _I64, _VP, _VP, _VP,
                                               ctypes.c_int, _VP, _VP, _SZ, ctypes.c_uint, _VP]),
}
EXPORTS = tuple(_SIGNATURES)

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblce.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LceError(f"{path} is missing: build it with `python -m vocab_projection_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().lce_status_string(status).decode()
        raise LceError(f"liblce call failed: {msg} ({status})")


def problem(n_tokens: int, hidden: int, vocab: int, dtype: torch.dtype, *,
            ignore_index: int = -100, reduction: str = "mean", strip: int = 0) -> Problem:
    if dtype not in _DTYPES:
        raise LceError(f"unsupported dtype {dtype}")
    if reduction not in _REDUCTIONS:
        raise LceError(f"unsupported reduction {reduction!r}")
    return Problem(n_tokens, hidden, vocab, strip or 0, _DTYPES[dtype], _REDUCTIONS[reduction],
                   ignore_index, 0)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---- the C entry points, one to one ----

def lce_pick_strip(p: Problem, budget_bytes: int) -> int:
    return int(load().lce_pick_strip(ctypes.byref(p), budget_bytes))


def lce_workspace_bytes(p: Problem) -> int:
    n = int(load().lce_workspace_bytes(ctypes.byref(p)))
    if n == 0:
        raise LceError("invalid problem")
    return n


def lce_forward_fold_max(p: Problem) -> int:
    n = int(load().lce_forward_fold_max(ctypes.byref(p)))
    if n < 0:
        raise LceError("invalid problem")
    return n


def lce_backward_fold_gemm_launches(p: Problem, v_len: int) -> int:
    n = int(load().lce_backward_fold_gemm_launches(ctypes.byref(p), v_len))
    if n < 0:
        raise LceError("invalid problem or strip length")
    return n


def lce_forward(p, hidden, weight, targets, loss, lse, row_loss, workspace, stream=None):
    _check(load().lce_forward(ctypes.byref(p), _ptr(hidden), _ptr(weight), _ptr(targets),
                              _ptr(loss), _ptr(lse), _ptr(row_loss), _ptr(workspace),
                              workspace.numel(), _stream(stream)))


def lce_backward(p, hidden, weight, targets, lse, grad_out, d_hidden, d_weight, workspace,
                 stream=None):
    _check(load().lce_backward(ctypes.byref(p), _ptr(hidden), _ptr(weight), _ptr(targets),
                               _ptr(lse), _ptr(grad_out), _ptr(d_hidden), _ptr(d_weight),
                               _ptr(workspace), workspace.numel(), _stream(stream)))


LCE_STATIC_SCRATCH_BYTES = 256 << 20


def lce_backward_static(p, hidden, weight, targets, lse, grad_out, d_hidden, d_weight,
                        stream=None):
    """lce_backward with the library's static per-GPU workspace (no workspace argument)."""
    _check(load().lce_backward_static(ctypes.byref(p), _ptr(hidden), _ptr(weight), _ptr(targets),
                                      _ptr(lse), _ptr(grad_out), _ptr(d_hidden), _ptr(d_weight),
                                      _stream(stream)))


def lce_forward_begin(p, workspace, stream=None):
    _check(load().lce_forward_begin(ctypes.byref(p), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))


def lce_forward_fold(p, hidden, weight_strip, v_begin, v_len, targets, workspace, stream=None):
    _check(load().lce_forward_fold(ctypes.byref(p), _ptr(hidden), _ptr(weight_strip), v_begin,
                                   v_len, _ptr(targets), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))


def lce_forward_end(p, targets, loss, lse, row_loss, workspace, stream=None):
    _check(load().lce_forward_end(ctypes.byref(p), _ptr(targets), _ptr(loss), _ptr(lse),
                                  _ptr(row_loss), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))


def lce_forward_state(p, state, workspace, stream=None):
    """Copy the running state into state (float32, 3 * N: max, sum, target logit)."""
    _check(load().lce_forward_state(ctypes.byref(p), _ptr(state), _ptr(workspace),
                                    workspace.numel(), _stream(stream)))


def lce_forward_merge_state(p, state, workspace, stream=None):
    """Fold a state exported by lce_forward_state (a disjoint vocabulary part) into workspace."""
    _check(load().lce_forward_merge_state(ctypes.byref(p), _ptr(state), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))


def lce_backward_begin(p, targets, grad_out, workspace, stream=None):
    _check(load().lce_backward_begin(ctypes.byref(p), _ptr(targets), _ptr(grad_out),
                                     _ptr(workspace), workspace.numel(), _stream(stream)))


def _acc_bits(accumulate, accumulate_dw):
    return (LCE_ACC_DHIDDEN if accumulate else 0) | (LCE_ACC_DWEIGHT if accumulate_dw else 0)


def lce_backward_fold(p, hidden, weight_strip, v_begin, v_len, targets, lse, d_hidden,
                      accumulate, d_weight_strip, workspace, stream=None, accumulate_dw=False):
    """accumulate: add to d_hidden; accumulate_dw: add to d_weight_strip."""
    _check(load().lce_backward_fold(ctypes.byref(p), _ptr(hidden), _ptr(weight_strip), v_begin,
                                    v_len, _ptr(targets), _ptr(lse), _ptr(d_hidden),
                                    _acc_bits(accumulate, accumulate_dw), _ptr(d_weight_strip),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))


def lce_forward_fold_steps(p, hidden, weight_strip, v_begin, v_len, targets, workspace, steps,
                           stream=None):
    _check(load().lce_forward_fold_steps(ctypes.byref(p), _ptr(hidden), _ptr(weight_strip),
                                         v_begin, v_len, _ptr(targets), _ptr(workspace),
                                         workspace.numel(), steps, _stream(stream)))


def lce_backward_fold_steps(p, hidden, weight_strip, v_begin, v_len, targets, lse, d_hidden,
                            accumulate, d_weight_strip, workspace, steps, stream=None,
                            accumulate_dw=False):
    _check(load().lce_backward_fold_steps(ctypes.byref(p), _ptr(hidden), _ptr(weight_strip),
                                          v_begin, v_len, _ptr(targets), _ptr(lse),
                                          _ptr(d_hidden), _acc_bits(accumulate, accumulate_dw),
                                          _ptr(d_weight_strip), _ptr(workspace),
                                          workspace.numel(), steps, _stream(stream)))


LCE_FUSED_ONE_SWEEP, LCE_FUSED_TWO_SWEEPS = 1, 2
FUSED_MODES = {"one_sweep": LCE_FUSED_ONE_SWEEP, "two_sweeps": LCE_FUSED_TWO_SWEEPS}


def lce_backward_fused_workspace_bytes(p: Problem, mode: int) -> int:
    n = int(load().lce_backward_fused_workspace_bytes(ctypes.byref(p), mode))
    if n == 0:
        raise LceError("invalid problem or mode")
    return n


def lce_backward_fused(p, hidden, weight, targets, lse, grad_out, d_hidden, d_weight, mode,
                       workspace, stream=None):
    """The backward without a strip buffer (mode LCE_FUSED_ONE_SWEEP or _TWO_SWEEPS)."""
    _check(load().lce_backward_fused(ctypes.byref(p), _ptr(hidden), _ptr(weight), _ptr(targets),
                                     _ptr(lse), _ptr(grad_out), _ptr(d_hidden), _ptr(d_weight),
                                     mode, _ptr(workspace), workspace.numel(), _stream(stream)))


LCE_ACC_NONE, LCE_ACC_DHIDDEN, LCE_ACC_DWEIGHT = 0, 1, 2
LCE_STEP_STRIP, LCE_STEP_MERGE = 1, 2
LCE_STEP_GRAD, LCE_STEP_DHIDDEN, LCE_STEP_DWEIGHT, LCE_STEP_ALL = 1, 2, 4, 7


# ---- torch-facing helpers ----

def _check_inputs(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor) -> None:
    if not (hidden.is_cuda and weight.is_cuda and targets.is_cuda):
        raise LceError("hidden, weight and targets must be GPU tensors")
    if hidden.dtype != weight.dtype or hidden.dtype not in _DTYPES:
        raise LceError("hidden and weight must share dtype float32 or bfloat16")
    if targets.dtype != torch.int32:
        raise LceError("targets must be int32")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise LceError("expected hidden [N, H] and weight [V, H]")
    if targets.shape != (hidden.shape[0],):
        raise LceError("targets must be [N]")
    for t in (hidden, weight, targets):
        if not t.is_contiguous():
            raise LceError("inputs must be contiguous")


def make_problem(hidden, weight, *, ignore_index=-100, reduction="mean", strip=0) -> Problem:
    return problem(hidden.shape[0], hidden.shape[1], weight.shape[0], hidden.dtype,
                   ignore_index=ignore_index, reduction=reduction, strip=strip)


def workspace(p: Problem, device) -> torch.Tensor:
    return torch.empty(lce_workspace_bytes(p), dtype=torch.uint8, device=device)


def forward(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor, *,
            ignore_index: int = -100, reduction: str = "mean", strip: int = 0,
            with_row_loss: bool = False, ws: Optional[torch.Tensor] = None):
    """(loss [1], lse [N]) or (loss, lse, row_loss) with with_row_loss."""
    _check_inputs(hidden, weight, targets)
    p = make_problem(hidden, weight, ignore_index=ignore_index, reduction=reduction, strip=strip)
    dev = hidden.device
    ws = workspace(p, dev) if ws is None else ws
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(hidden.shape[0], dtype=torch.float32, device=dev)
    row_loss = torch.empty_like(lse) if with_row_loss else None
    lce_forward(p, hidden, weight, targets, loss, lse, row_loss, ws)
    return (loss, lse, row_loss) if with_row_loss else (loss, lse)


def backward(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
             lse: torch.Tensor, grad_out: torch.Tensor, *, ignore_index: int = -100,
             reduction: str = "mean", strip: int = 0, ws: Optional[torch.Tensor] = None):
    """(d_hidden [N, H] float32, d_weight [V, H] float32)."""
    _check_inputs(hidden, weight, targets)
    p = make_problem(hidden, weight, ignore_index=ignore_index, reduction=reduction, strip=strip)
    dev = hidden.device
    ws = workspace(p, dev) if ws is None else ws
    go = grad_out.reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    d_hidden = torch.empty(hidden.shape, dtype=torch.float32, device=dev)
    d_weight = torch.empty(weight.shape, dtype=torch.float32, device=dev)
    lce_backward(p, hidden, weight, targets, lse.contiguous(), go, d_hidden, d_weight, ws)
    return d_hidden, d_weight


class LinearCrossEntropy(torch.autograd.Function):
    """loss = CE(hidden . weight^T, targets) with the strip-wise HIP kernels.

    Saves only lse [N] for the backward pass, which recomputes the logits.
    The gradients are float32 and are cast to the inputs' dtype.
    """

    @staticmethod
    def forward(ctx, hidden, weight, targets, ignore_index=-100, reduction="mean", strip=0):
        loss, lse = forward(hidden, weight, targets, ignore_index=ignore_index,
                            reduction=reduction, strip=strip)
        ctx.save_for_backward(hidden, weight, targets, lse)
        ctx.cfg = (ignore_index, reduction, strip)
        return loss[0]

    @staticmethod
    def backward(ctx, grad_loss):
        hidden, weight, targets, lse = ctx.saved_tensors
        ignore_index, reduction, strip = ctx.cfg
        dh, dw = backward(hidden, weight, targets, lse, grad_loss, ignore_index=ignore_index,
                          reduction=reduction, strip=strip)
        return dh.to(hidden.dtype), dw.to(weight.dtype), None, None, None, None
