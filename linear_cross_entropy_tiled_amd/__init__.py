"""Fused linear cross-entropy for AMD MI355X (gfx950): Python binding.

The compute lives in ``libflce.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/flce.h``).  This module only marshals arguments:

* ``flce_workspace_size``, ``flce_forward``, ``flce_backward``,
  ``flce_get_status``, ``flce_status_string``, ``flce_version`` mirror the C
  entry points one to one and take raw device pointers (ints);
* ``forward`` / ``backward`` are torch conveniences that allocate outputs and
  the workspace with torch and pass the current HIP stream;
* ``chunked_linear_loss`` / ``weighted_mse`` drive the generic chunked loss
  (``flce_chunked_linear_loss``) with a Python loss function or the built-in
  weighted squared error (``flce_weighted_mse_chunk``).

There is no fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libflce.so")

FLCE_OK = 0
FLCE_ERR_INVALID_ARG = -1
FLCE_ERR_UNSUPPORTED = -2
FLCE_ERR_WORKSPACE_TOO_SMALL = -3
FLCE_ERR_HIP = -4
FLCE_ERR_TARGET_OUT_OF_RANGE = -5
FLCE_ERR_CALLBACK = -6

FLCE_F32 = 0
FLCE_BF16 = 1
FLCE_F16 = 2
DTYPES = {"f32": FLCE_F32, "bf16": FLCE_BF16, "f16": FLCE_F16}
REDUCTIONS = {"none": 0, "sum": 1, "mean": 2}
FLCE_PASS_FORWARD = 0
FLCE_PASS_BACKWARD = 1
FLCE_ACCUMULATE_GRAD_WEIGHT = 1
FLCE_ACCUMULATE_GRAD_BIAS = 2
FLCE_TARGETS_INT32 = 4
FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT = 8

EXPORTED = ("flce_workspace_size", "flce_forward", "flce_backward", "flce_get_status",
            "flce_status_string", "flce_version", "flce_chunked_workspace_size",
            "flce_chunked_linear_loss", "flce_weighted_mse_chunk", "flce_forward_backward_workspace_size",
            "flce_forward_backward", "flce_scale_gradients", "flce_forward_timed", "flce_backward_timed",
            "flce_forward_no_alloc")

FLCE_KERNEL_FORWARD_TILES = 1
FLCE_KERNEL_DLOGITS = 2
FLCE_KERNEL_GRAD_WEIGHT = 3
FLCE_KERNEL_GRAD_HIDDEN = 4
KERNEL_NAMES = {FLCE_KERNEL_FORWARD_TILES: "fwd_tiles_kernel", FLCE_KERNEL_DLOGITS: "bwd_dlogits_kernel",
                FLCE_KERNEL_GRAD_WEIGHT: "bwd_gw_kernel", FLCE_KERNEL_GRAD_HIDDEN: "bwd_gh_kernel"}


class flce_params(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("ignore_index", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("grad_weight_dtype", ctypes.c_int32),
        ("reduction", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("logit_scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("z_loss", ctypes.c_float),
        ("reserved_f", ctypes.c_float),
        ("vocab_chunk", ctypes.c_int64),
    ]


class flce_launch_timer(ctypes.Structure):
    _fields_ = [
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("kernel", ctypes.POINTER(ctypes.c_int32)),
        ("capacity", ctypes.c_int32),
        ("count", ctypes.c_int32),
    ]


class flce_chunked_params(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("chunk_rows", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("grad_weight_dtype", ctypes.c_int32),
        ("accum_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class flce_wmse_args(ctypes.Structure):
    _fields_ = [
        ("target", ctypes.c_void_p),
        ("ld_target", ctypes.c_int64),
        ("row_weight", ctypes.c_void_p),
        ("feature_weight", ctypes.c_void_p),
        ("row_loss", ctypes.c_void_p),
    ]


# int fn(void* user, int64 row0, int64 rows, int64 vocab, void* logits, int64 ld, int32 dtype,
#        float* loss, void* stream)
CHUNK_LOSS_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p)


class FlceError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {status_string(code)} ({code})")
        self.code = code


_lib = None


def load(path: Optional[str] = None):
    """Load libflce.so (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    # FLCE_LIB_PATH: another build of the same library (the host-sanitizer build of
    # linear_cross_entropy_tiled_amd.build --host-sanitizers), for the host-side tests
    path = path or os.environ.get("FLCE_LIB_PATH") or LIB_PATH
    # torch first: the library links the HIP runtime by soname, and the copy
    # torch ships must be the one in the process (a second runtime loaded
    # ahead of torch's crashes it)
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m linear_cross_entropy_tiled_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(flce_params)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.flce_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
    lib.flce_workspace_size.restype = ctypes.c_int
    lib.flce_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.flce_forward.restype = ctypes.c_int
    lib.flce_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.flce_backward.restype = ctypes.c_int
    lib.flce_get_status.argtypes = [vp, vp]
    lib.flce_get_status.restype = ctypes.c_int
    lib.flce_status_string.argtypes = [ctypes.c_int]
    lib.flce_status_string.restype = ctypes.c_char_p
    lib.flce_version.argtypes = []
    lib.flce_version.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.flce_forward_backward_workspace_size.argtypes = [P, i64, ctypes.POINTER(sz)]
    lib.flce_forward_backward_workspace_size.restype = ctypes.c_int
    lib.flce_forward_backward.argtypes = [P, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.flce_forward_backward.restype = ctypes.c_int
    TP = ctypes.POINTER(flce_launch_timer)
    lib.flce_forward_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, TP]
    lib.flce_forward_timed.restype = ctypes.c_int
    lib.flce_backward_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, TP]
    lib.flce_backward_timed.restype = ctypes.c_int
    lib.flce_forward_no_alloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.flce_forward_no_alloc.restype = ctypes.c_int
    lib.flce_scale_gradients.argtypes = [P, vp, vp, vp, vp, vp]
    lib.flce_scale_gradients.restype = ctypes.c_int
    CP = ctypes.POINTER(flce_chunked_params)
    lib.flce_chunked_workspace_size.argtypes = [CP, ctypes.POINTER(sz)]
    lib.flce_chunked_workspace_size.restype = ctypes.c_int
    lib.flce_chunked_linear_loss.argtypes = [CP, vp, vp, CHUNK_LOSS_FN, vp, vp, vp, vp, vp, sz, vp]
    lib.flce_chunked_linear_loss.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.flce_weighted_mse_chunk.argtypes = [vp, i64, i64, i64, vp, i64, ctypes.c_int32, vp, vp]
    lib.flce_weighted_mse_chunk.restype = ctypes.c_int
    _lib = lib
    return lib


# ----------------------------------------------------------------------------- raw C entry points

def flce_workspace_size(params: flce_params, pass_: int) -> int:
    out = ctypes.c_size_t(0)
    rc = load().flce_workspace_size(ctypes.byref(params), pass_, ctypes.byref(out))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_workspace_size")
    return out.value


def flce_forward(params, hidden, weight, bias, targets, loss, lse, num_correct, entropy_sum,
                 workspace, workspace_bytes, stream) -> int:
    return load().flce_forward(ctypes.byref(params), hidden, weight, bias, targets, loss, lse,
                               num_correct, entropy_sum, workspace, workspace_bytes, stream)


def flce_backward(params, hidden, weight, bias, targets, lse, grad_loss, grad_hidden, grad_weight,
                  grad_bias, workspace, workspace_bytes, stream) -> int:
    return load().flce_backward(ctypes.byref(params), hidden, weight, bias, targets, lse, grad_loss,
                                grad_hidden, grad_weight, grad_bias, workspace, workspace_bytes,
                                stream)


def flce_forward_timed(params, hidden, weight, bias, targets, loss, lse, num_correct, entropy_sum,
                       workspace, workspace_bytes, stream, timer) -> int:
    return load().flce_forward_timed(ctypes.byref(params), hidden, weight, bias, targets, loss, lse,
                                     num_correct, entropy_sum, workspace, workspace_bytes, stream,
                                     None if timer is None else ctypes.byref(timer))


def flce_backward_timed(params, hidden, weight, bias, targets, lse, grad_loss, grad_hidden, grad_weight,
                        grad_bias, workspace, workspace_bytes, stream, timer) -> int:
    return load().flce_backward_timed(ctypes.byref(params), hidden, weight, bias, targets, lse, grad_loss,
                                      grad_hidden, grad_weight, grad_bias, workspace, workspace_bytes, stream,
                                      None if timer is None else ctypes.byref(timer))


class LaunchTimer:
    """Host side of flce_launch_timer: `capacity` pairs of caller-owned HIP events (torch
    events, recorded once on `stream` so that they exist) that flce_forward_timed /
    flce_backward_timed record around their matrix-core launches.  ``durations()`` maps
    each kernel name to the milliseconds of its timed launches, after a synchronize."""

    def __init__(self, capacity: int, stream):
        import torch
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * capacity)]
        for e in self.events:
            e.record(stream)
        handles = [e.cuda_event for e in self.events]
        if not all(handles):
            raise RuntimeError("torch did not create the timing events")
        self._handles = (ctypes.c_void_p * len(handles))(*handles)
        self._kinds = (ctypes.c_int32 * capacity)()
        self.c = flce_launch_timer(ctypes.cast(self._handles, ctypes.POINTER(ctypes.c_void_p)),
                                   ctypes.cast(self._kinds, ctypes.POINTER(ctypes.c_int32)), capacity, 0)

    def reset(self):
        self.c.count = 0

    def durations(self):
        out = {}
        for k in range(self.c.count):
            ms = self.events[2 * k].elapsed_time(self.events[2 * k + 1])
            out.setdefault(KERNEL_NAMES.get(self._kinds[k], str(self._kinds[k])), []).append(ms)
        return out


def flce_forward_no_alloc(params, hidden, weight, bias, targets, loss, lse, num_correct, entropy_sum,
                          stream) -> int:
    return load().flce_forward_no_alloc(ctypes.byref(params), hidden, weight, bias, targets, loss, lse,
                                        num_correct, entropy_sum, stream)


def flce_forward_backward_workspace_size(params: flce_params, block_rows: int = 0) -> int:
    out = ctypes.c_size_t(0)
    rc = load().flce_forward_backward_workspace_size(ctypes.byref(params), block_rows, ctypes.byref(out))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward_backward_workspace_size")
    return out.value


def flce_forward_backward(params, block_rows, hidden, weight, bias, targets, grad_loss, loss, lse, num_correct,
                          entropy_sum, grad_hidden, grad_weight, grad_bias, workspace, workspace_bytes,
                          stream) -> int:
    return load().flce_forward_backward(ctypes.byref(params), block_rows, hidden, weight, bias, targets, grad_loss,
                                        loss, lse, num_correct, entropy_sum, grad_hidden, grad_weight, grad_bias,
                                        workspace, workspace_bytes, stream)


def flce_scale_gradients(params, g, grad_hidden, grad_weight, grad_bias, stream) -> int:
    return load().flce_scale_gradients(ctypes.byref(params), g, grad_hidden, grad_weight, grad_bias, stream)


def flce_chunked_workspace_size(params: flce_chunked_params) -> int:
    out = ctypes.c_size_t(0)
    rc = load().flce_chunked_workspace_size(ctypes.byref(params), ctypes.byref(out))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_chunked_workspace_size")
    return out.value


def flce_chunked_linear_loss(params, inputs, weight, fn, user, loss, grad_inputs, grad_weight, workspace,
                             workspace_bytes, stream) -> int:
    return load().flce_chunked_linear_loss(ctypes.byref(params), inputs, weight, fn, user, loss, grad_inputs,
                                           grad_weight, workspace, workspace_bytes, stream)


def weighted_mse_chunk_fn():
    """The library's built-in loss function (flce_weighted_mse_chunk) as a CHUNK_LOSS_FN."""
    return ctypes.cast(load().flce_weighted_mse_chunk, CHUNK_LOSS_FN)


def flce_get_status(workspace, stream) -> int:
    return load().flce_get_status(workspace, stream)


def flce_status_string(code: int) -> str:
    return load().flce_status_string(code).decode()


def flce_version() -> int:
    return load().flce_version()


def status_string(code: int) -> str:
    try:
        return flce_status_string(code)
    except Exception:
        return "status"


# ----------------------------------------------------------------------------- torch conveniences

def make_params(n_tokens: int, hidden: int, vocab: int, *, dtype: str = "bf16",
                grad_weight_dtype: Optional[str] = None, logit_scale: float = 1.0,
                softcap: Optional[float] = None, z_loss: float = 0.0, ignore_index: int = -100,
                reduction: str = "mean", accumulate_grad_weight: bool = False,
                accumulate_grad_bias: bool = False, targets_int32: bool = False,
                grad_weight_accum_dtype: str = "fp32", vocab_chunk: int = 0) -> flce_params:
    if reduction not in REDUCTIONS:
        raise ValueError(f"invalid reduction {reduction!r}")
    dt = DTYPES
    p = flce_params()
    p.n_tokens, p.hidden, p.vocab, p.ignore_index = n_tokens, hidden, vocab, ignore_index
    p.dtype = dt[dtype]
    p.grad_weight_dtype = dt[grad_weight_dtype or dtype]
    p.reduction = REDUCTIONS[reduction]
    p.logit_scale = logit_scale
    p.softcap = softcap if softcap else 0.0
    p.z_loss = z_loss
    p.vocab_chunk = vocab_chunk
    p.flags = (FLCE_ACCUMULATE_GRAD_WEIGHT if accumulate_grad_weight else 0) | \
              (FLCE_ACCUMULATE_GRAD_BIAS if accumulate_grad_bias else 0) | \
              (FLCE_TARGETS_INT32 if targets_int32 else 0)
    if grad_weight_accum_dtype not in ("fp32", "weight"):
        raise ValueError(f"invalid grad_weight_accum_dtype {grad_weight_accum_dtype!r}")
    if grad_weight_accum_dtype == "weight":
        p.flags |= FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT
    return p


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_name(t) -> str:
    import torch
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float16:
        return "f16"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {t.dtype}")


def _targets_int32(t) -> bool:
    import torch
    if t.dtype == torch.int64:
        return False
    if t.dtype == torch.int32:
        return True
    raise TypeError(f"targets must be int64 or int32, not {t.dtype}")


def _check(t, name):
    if t is not None and (not t.is_cuda or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")


def _validate(hidden, weight, targets, bias=None, *, reduction="mean", lse=None, grad_loss=None,
              grad_weight=None, grad_bias=None):
    """Host-side checks before anything is launched.  The kernels read weight and bias in
    hidden's dtype with hidden's row length, targets, lse and the upstream gradient with the
    lengths N implies, and the gradient buffers with the weight's shape; a mismatch would read
    or write out of bounds (or silently misread), so it raises TypeError (types) or
    ValueError (shapes, layout, devices) here instead."""
    import torch
    if reduction not in REDUCTIONS:
        raise ValueError(f"invalid reduction {reduction!r}")
    if hidden.dim() != 2 or weight.dim() != 2:
        raise ValueError(f"hidden and weight must be 2-D, got {tuple(hidden.shape)} and {tuple(weight.shape)}")
    dt = _dtype_name(hidden)
    n, h = hidden.shape
    v = weight.shape[0]
    if weight.dtype != hidden.dtype:
        raise TypeError(f"weight dtype {weight.dtype} differs from hidden's {hidden.dtype}")
    if weight.shape[1] != h:
        raise ValueError(f"weight has {weight.shape[1]} columns, hidden has {h}")
    if bias is not None:
        if bias.dtype != hidden.dtype:
            raise TypeError(f"bias dtype {bias.dtype} differs from hidden's {hidden.dtype}")
        if bias.dim() != 1 or bias.shape[0] != v:
            raise ValueError(f"bias must have shape ({v},), got {tuple(bias.shape)}")
    _targets_int32(targets)
    if targets.dim() != 1 or targets.shape[0] != n:
        raise ValueError(f"targets must have shape ({n},), got {tuple(targets.shape)}")
    if lse is not None:
        if lse.dtype != torch.float32:
            raise TypeError(f"lse must be float32, not {lse.dtype}")
        if lse.numel() != n:
            raise ValueError(f"lse must hold {n} values, got {lse.numel()}")
    if grad_loss is not None:
        if grad_loss.dtype != torch.float32:
            raise TypeError(f"grad_loss must be float32, not {grad_loss.dtype}")
        want = n if reduction == "none" else 1
        if grad_loss.numel() != want and not (reduction == "none" and n == 0):
            raise ValueError(f"grad_loss must hold {want} value(s) for reduction {reduction!r}, "
                             f"got {grad_loss.numel()}")
    if grad_weight is not None:
        _dtype_name(grad_weight)
        if tuple(grad_weight.shape) != (v, h):
            raise ValueError(f"grad_weight must have the weight's shape {(v, h)}, got {tuple(grad_weight.shape)}")
    if grad_bias is not None:
        if bias is None:
            raise ValueError("grad_bias needs a bias")
        if grad_bias.dtype != bias.dtype:
            raise TypeError(f"grad_bias dtype {grad_bias.dtype} differs from bias's {bias.dtype}")
        if tuple(grad_bias.shape) != (v,):
            raise ValueError(f"grad_bias must have shape ({v},), got {tuple(grad_bias.shape)}")
    named = [("hidden", hidden), ("weight", weight), ("targets", targets), ("bias", bias), ("lse", lse),
             ("grad_loss", grad_loss), ("grad_weight", grad_weight), ("grad_bias", grad_bias)]
    for name, t in named:
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t in named:
        if t is not None and (t.device.type != "cuda" or t.device != hidden.device):
            raise ValueError(f"{name} must be on hidden's GPU ({hidden.device}), not {t.device}")
    return dt


def forward(hidden, weight, targets, bias=None, *, logit_scale: float = 1.0,
            softcap: Optional[float] = None, z_loss: float = 0.0, ignore_index: int = -100,
            reduction: str = "mean", return_metrics: bool = False, workspace=None):
    """Runs flce_forward on the current stream.  Returns (loss, lse, metrics | None)."""
    import torch
    dt = _validate(hidden, weight, targets, bias, reduction=reduction)
    n, h = hidden.shape
    v = weight.shape[0]
    p = make_params(n, h, v, dtype=dt, logit_scale=logit_scale, softcap=softcap,
                    z_loss=z_loss, ignore_index=ignore_index, reduction=reduction,
                    targets_int32=_targets_int32(targets))
    dev = hidden.device
    ws_bytes = flce_workspace_size(p, FLCE_PASS_FORWARD)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss = torch.empty(n if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    nc = torch.empty(1, dtype=torch.int64, device=dev) if return_metrics else None
    ent = torch.empty(1, dtype=torch.float32, device=dev) if return_metrics else None
    rc = flce_forward(p, _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets), _ptr(loss), _ptr(lse),
                      _ptr(nc), _ptr(ent), _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward")
    if reduction != "none":
        loss = loss.reshape(())
    metrics = {"num_correct_tokens": nc.reshape(()), "entropy_sum": ent.reshape(())} if return_metrics else None
    return loss, lse, metrics


def backward(hidden, weight, targets, lse, grad_loss, bias=None, *, logit_scale: float = 1.0,
             softcap: Optional[float] = None, z_loss: float = 0.0, ignore_index: int = -100,
             reduction: str = "mean", grad_weight_dtype: Optional[str] = None, workspace=None,
             grad_weight=None, grad_bias=None, vocab_chunk: int = 0):
    """Runs flce_backward on the current stream.  Returns (grad_hidden, grad_weight, grad_bias).

    If ``grad_weight`` (``grad_bias``) is given, the gradient is added to it in place (the
    FLCE_ACCUMULATE_GRAD_WEIGHT / _BIAS flags) and the same tensor is returned.
    ``vocab_chunk``: vocabulary rows per chunk of the logit-gradient scratch (a multiple of
    256; 0 = the library's choice)."""
    import torch
    dt = _validate(hidden, weight, targets, bias, reduction=reduction, lse=lse, grad_loss=grad_loss,
                   grad_weight=grad_weight, grad_bias=grad_bias)
    n, h = hidden.shape
    v = weight.shape[0]
    if grad_weight is not None:
        grad_weight_dtype = _dtype_name(grad_weight)
    p = make_params(n, h, v, dtype=dt, grad_weight_dtype=grad_weight_dtype, logit_scale=logit_scale,
                    softcap=softcap, z_loss=z_loss, ignore_index=ignore_index, reduction=reduction,
                    accumulate_grad_weight=grad_weight is not None, accumulate_grad_bias=grad_bias is not None,
                    targets_int32=_targets_int32(targets), vocab_chunk=vocab_chunk)
    dev = hidden.device
    ws_bytes = flce_workspace_size(p, FLCE_PASS_BACKWARD)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    gh = torch.empty((n, h), dtype=hidden.dtype, device=dev)
    gw = grad_weight if grad_weight is not None else torch.empty((v, h), dtype=tdt[grad_weight_dtype or dt], device=dev)
    gb = grad_bias if grad_bias is not None else (torch.empty(v, dtype=bias.dtype, device=dev) if bias is not None else None)
    rc = flce_backward(p, _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets), _ptr(lse),
                       _ptr(grad_loss), _ptr(gh), _ptr(gw), _ptr(gb), _ptr(workspace),
                       workspace.numel(), _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_backward")
    return gh, gw, gb


def forward_backward(hidden, weight, targets, grad_loss, bias=None, *, logit_scale: float = 1.0,
                     softcap: Optional[float] = None, z_loss: float = 0.0, ignore_index: int = -100,
                     reduction: str = "mean", grad_weight_dtype: Optional[str] = None, return_metrics: bool = False,
                     block_rows: int = 0, grad_weight_accum_dtype: str = "fp32", workspace=None, grad_weight=None,
                     grad_bias=None):
    """Runs flce_forward_backward (loss and gradients in one pass, the upstream gradient
    ``grad_loss`` given up front) on the current stream.  Returns
    (loss, lse, metrics | None, grad_hidden, grad_weight, grad_bias); ``grad_weight`` /
    ``grad_bias`` given: accumulated into in place, as in ``backward``.  ``grad_weight_accum_dtype``:
    "fp32" (sum over the row blocks in fp32, round once) or "weight" (sum in grad_weight's dtype)."""
    import torch
    dt = _validate(hidden, weight, targets, bias, reduction=reduction, grad_loss=grad_loss,
                   grad_weight=grad_weight, grad_bias=grad_bias)
    n, h = hidden.shape
    v = weight.shape[0]
    if grad_weight is not None:
        grad_weight_dtype = _dtype_name(grad_weight)
    p = make_params(n, h, v, dtype=dt, grad_weight_dtype=grad_weight_dtype, logit_scale=logit_scale,
                    softcap=softcap, z_loss=z_loss, ignore_index=ignore_index, reduction=reduction,
                    accumulate_grad_weight=grad_weight is not None, accumulate_grad_bias=grad_bias is not None,
                    targets_int32=_targets_int32(targets), grad_weight_accum_dtype=grad_weight_accum_dtype)
    dev = hidden.device
    ws_bytes = flce_forward_backward_workspace_size(p, block_rows)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    loss = torch.empty(n if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    nc = torch.empty(1, dtype=torch.int64, device=dev) if return_metrics else None
    ent = torch.empty(1, dtype=torch.float32, device=dev) if return_metrics else None
    gh = torch.empty((n, h), dtype=hidden.dtype, device=dev)
    gw = grad_weight if grad_weight is not None else torch.empty((v, h), dtype=tdt[grad_weight_dtype or dt], device=dev)
    gb = grad_bias if grad_bias is not None else (torch.empty(v, dtype=bias.dtype, device=dev) if bias is not None else None)
    rc = flce_forward_backward(p, block_rows, _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets), _ptr(grad_loss),
                               _ptr(loss), _ptr(lse), _ptr(nc), _ptr(ent), _ptr(gh), _ptr(gw), _ptr(gb),
                               _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_forward_backward")
    if reduction != "none":
        loss = loss.reshape(())
    metrics = {"num_correct_tokens": nc.reshape(()), "entropy_sum": ent.reshape(())} if return_metrics else None
    return loss, lse, metrics, gh, gw, gb


def linear_cross_entropy(hidden, weight, targets, bias=None, *, logit_scale: float = 1.0,
                         softcap: Optional[float] = None, z_loss: float = 0.0, ignore_index: int = -100,
                         reduction: str = "mean", one_pass: bool = False):
    """The loss as a differentiable torch op.  Returns the loss (a scalar, or (N,) for "none").

    one_pass=False: flce_forward now, flce_backward (which recomputes the logit tiles from
    hidden, weight and the saved LSE) when autograd asks for gradients, with the upstream
    gradient autograd supplies.
    one_pass=True ("sum" / "mean" only): flce_forward_backward now, with an upstream gradient
    of 1, keeping the gradients; autograd's backward multiplies them by the upstream scalar
    (flce_scale_gradients), once: the graph cannot be backpropagated a second time."""
    import torch

    opts = dict(logit_scale=logit_scale, softcap=softcap, z_loss=z_loss, ignore_index=ignore_index,
                reduction=reduction)
    if one_pass:
        if reduction == "none":
            raise ValueError('one_pass needs reduction "sum" or "mean": the per-row upstream gradient of '
                             '"none" must be known before the pass (use forward_backward)')

        class _OnePass(torch.autograd.Function):
            @staticmethod
            def forward(ctx, x, w, b):
                one = torch.ones(1, dtype=torch.float32, device=x.device)
                loss, _, _, gh, gw, gb = forward_backward(x, w, targets, one, b, **opts)
                p = make_params(x.shape[0], x.shape[1], w.shape[0], dtype=_dtype_name(x), **opts)
                ctx.state = [p, gh, gw, gb]
                return loss

            @staticmethod
            def backward(ctx, g):
                if ctx.state is None:
                    raise RuntimeError("the one-pass linear_cross_entropy gradients were already used")
                p, gh, gw, gb = ctx.state
                ctx.state = None
                g = g.detach().to(torch.float32).contiguous().reshape(1)
                rc = flce_scale_gradients(p, _ptr(g), _ptr(gh), _ptr(gw), _ptr(gb), _stream_handle(g.device))
                if rc != FLCE_OK:
                    raise FlceError(rc, "flce_scale_gradients")
                return gh, gw, gb

        return _OnePass.apply(hidden, weight, bias)

    class _Fn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w, b):
            loss, lse, _ = forward(x, w, targets, b, **opts)
            ctx.save_for_backward(x, w, b, lse)
            return loss

        @staticmethod
        def backward(ctx, g):
            x, w, b, lse = ctx.saved_tensors
            g = g.detach().to(torch.float32).contiguous().reshape(-1)
            gh, gw, gb = backward(x, w, targets, lse, g, b, **opts)   # gradients in the inputs' dtypes
            return gh, gw, gb

    return _Fn.apply(hidden, weight, bias)


def get_status(workspace) -> int:
    return flce_get_status(_ptr(workspace), _stream_handle(workspace.device))


# ----------------------------------------------------------------------------- generic chunked loss

def make_chunked_params(n_tokens: int, hidden: int, vocab: int, *, dtype: str = "bf16",
                        grad_weight_dtype: Optional[str] = None, grad_weight_accum_dtype: str = "fp32",
                        chunk_rows: int = 0, accumulate_grad_weight: bool = False) -> flce_chunked_params:
    if grad_weight_accum_dtype not in ("fp32", "weight"):
        raise ValueError(f"invalid grad_weight_accum_dtype {grad_weight_accum_dtype!r}")
    p = flce_chunked_params()
    p.n_tokens, p.hidden, p.vocab, p.chunk_rows = n_tokens, hidden, vocab, chunk_rows
    p.dtype = DTYPES[dtype]
    p.grad_weight_dtype = DTYPES[grad_weight_dtype or dtype]
    p.accum_dtype = FLCE_F32 if grad_weight_accum_dtype == "fp32" else p.grad_weight_dtype
    p.flags = FLCE_ACCUMULATE_GRAD_WEIGHT if accumulate_grad_weight else 0
    return p


def _run_chunked(inputs, weight, fn, user, *, chunk_rows, grad_weight_dtype, grad_weight_accum_dtype,
                 grad_weight, workspace, on_error=None):
    import torch
    if inputs.dim() != 2 or weight.dim() != 2:
        raise ValueError(f"inputs and weight must be 2-D, got {tuple(inputs.shape)} and {tuple(weight.shape)}")
    n, h = inputs.shape
    v = weight.shape[0]
    dt = _dtype_name(inputs)
    if weight.dtype != inputs.dtype:
        raise TypeError(f"weight dtype {weight.dtype} differs from the inputs' {inputs.dtype}")
    if weight.shape[1] != h:
        raise ValueError(f"weight has {weight.shape[1]} columns, inputs have {h}")
    if grad_weight is not None:
        grad_weight_dtype = _dtype_name(grad_weight)
        if tuple(grad_weight.shape) != (v, h):
            raise ValueError("grad_weight must have the weight's shape")
    for t, nme in ((inputs, "inputs"), (weight, "weight"), (grad_weight, "grad_weight")):
        _check(t, nme)
        if t is not None and t.device != inputs.device:
            raise ValueError(f"{nme} must be on the inputs' GPU")
    p = make_chunked_params(n, h, v, dtype=dt, grad_weight_dtype=grad_weight_dtype,
                            grad_weight_accum_dtype=grad_weight_accum_dtype, chunk_rows=chunk_rows,
                            accumulate_grad_weight=grad_weight is not None)
    dev = inputs.device
    ws_bytes = flce_chunked_workspace_size(p)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    gi = torch.empty((n, h), dtype=inputs.dtype, device=dev)
    gw = grad_weight if grad_weight is not None else torch.empty((v, h), dtype=tdt[grad_weight_dtype or dt], device=dev)
    rc = flce_chunked_linear_loss(p, _ptr(inputs), _ptr(weight), fn, user, _ptr(loss), _ptr(gi), _ptr(gw),
                                  _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if rc == FLCE_ERR_CALLBACK and on_error is not None and on_error[0] is not None:
        raise on_error[0]
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_chunked_linear_loss")
    return loss.reshape(()), gi, gw


def chunked_linear_loss(inputs, weight, loss_and_grad_fn, *args, chunk_rows: int = 0,
                        grad_weight_dtype: Optional[str] = None, grad_weight_accum_dtype: str = "fp32",
                        grad_weight=None, workspace=None, **kwargs):
    """Generic chunked linear loss with a Python loss function.

    ``loss_and_grad_fn(logits_chunk, *chunk_args, **chunk_kwargs) -> (loss, grad_logits)`` sees one
    block of rows of ``inputs @ weight.T`` (in the inputs' dtype) and returns the block's scalar loss
    and the gradient of the logits (same shape).  Tensor arguments whose leading dimension is N are
    sliced to the block's rows; others are passed through.  Returns (loss, grad_inputs, grad_weight);
    with ``grad_weight`` given, the weight gradient is added to it in place."""
    import torch
    n = inputs.shape[0]
    ws_holder = {}
    err = [None]

    def slice_arg(a, r0, rows):
        if isinstance(a, torch.Tensor) and a.dim() > 0 and a.shape[0] == n:
            return a[r0:r0 + rows]
        return a

    def cb(user, row0, rows, vocab, logits_ptr, ld, dtype, loss_ptr, stream):
        try:
            ws = ws_holder["ws"]
            esize = 4 if dtype == FLCE_F32 else 2
            off = logits_ptr - ws.data_ptr()
            tdt = {FLCE_F32: torch.float32, FLCE_BF16: torch.bfloat16, FLCE_F16: torch.float16}[dtype]
            buf = ws[off:off + rows * ld * esize].view(tdt).view(rows, ld)[:, :vocab]
            c_args = [slice_arg(a, row0, rows) for a in args]
            c_kwargs = {k: slice_arg(a, row0, rows) for k, a in kwargs.items()}
            loss, grad = loss_and_grad_fn(buf, *c_args, **c_kwargs)
            buf.copy_(grad)
            ws_holder["loss"].add_(loss.reshape(1).to(torch.float32))
            return 0
        except Exception as e:   # reported after the library returns
            err[0] = e
            return 1

    fn = CHUNK_LOSS_FN(cb)
    h = inputs.shape[1]
    v = weight.shape[0]
    p = make_chunked_params(n, h, v, dtype=_dtype_name(inputs), grad_weight_dtype=grad_weight_dtype,
                            grad_weight_accum_dtype=grad_weight_accum_dtype, chunk_rows=chunk_rows)
    ws_bytes = flce_chunked_workspace_size(p)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=inputs.device)
    ws_holder["ws"] = workspace
    # the callback adds each block's loss to a torch scalar; the library's own loss word is unused
    ws_holder["loss"] = torch.zeros(1, dtype=torch.float32, device=inputs.device)
    _, gi, gw = _run_chunked(inputs, weight, fn, None, chunk_rows=chunk_rows, grad_weight_dtype=grad_weight_dtype,
                             grad_weight_accum_dtype=grad_weight_accum_dtype, grad_weight=grad_weight,
                             workspace=workspace, on_error=err)
    return ws_holder["loss"].reshape(()), gi, gw


def weighted_mse(inputs, weight, target, row_weight, feature_weight, *, chunk_rows: int = 0,
                 grad_weight_dtype: Optional[str] = None, grad_weight_accum_dtype: str = "fp32",
                 grad_weight=None, workspace=None):
    """Generic chunked linear loss with the built-in weighted squared error:
    loss = sum_ij (z_ij - target_ij)^2 row_weight_i feature_weight_j, z = inputs @ weight.T.
    ``target`` is (N, V) fp32 with contiguous rows, the weights fp32 vectors."""
    import torch
    if weight.dtype != inputs.dtype:
        raise TypeError(f"weight dtype {weight.dtype} differs from the inputs' {inputs.dtype}")
    for t, nme in ((target, "target"), (row_weight, "row_weight"), (feature_weight, "feature_weight")):
        if t.dtype != torch.float32:
            raise TypeError(f"{nme} must be float32, not {t.dtype}")
        if t.device != inputs.device or not t.is_cuda:
            raise ValueError(f"{nme} must be on the inputs' GPU")
    if target.stride(1) != 1 or not row_weight.is_contiguous() or not feature_weight.is_contiguous():
        raise ValueError("target rows, row_weight and feature_weight must be contiguous")
    n, v = inputs.shape[0], weight.shape[0]
    if target.dim() != 2 or target.shape[0] != n or target.shape[1] != v:
        raise ValueError(f"target must have shape ({n}, {v}), got {tuple(target.shape)}")
    if row_weight.numel() != n or feature_weight.numel() != v:
        raise ValueError(f"row_weight must hold {n} values and feature_weight {v}")
    row_loss = torch.empty(inputs.shape[0], dtype=torch.float32, device=inputs.device)
    a = flce_wmse_args(_ptr(target), target.stride(0), _ptr(row_weight), _ptr(feature_weight), _ptr(row_loss))
    return _run_chunked(inputs, weight, weighted_mse_chunk_fn(), ctypes.cast(ctypes.pointer(a), ctypes.c_void_p),
                        chunk_rows=chunk_rows, grad_weight_dtype=grad_weight_dtype,
                        grad_weight_accum_dtype=grad_weight_accum_dtype, grad_weight=grad_weight,
                        workspace=workspace)
