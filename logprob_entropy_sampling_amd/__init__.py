"""Vocabulary-scale LM-head scoring on MI355X: thin Python binding of libvocabscore.so.

Argument marshalling only: tensors are checked, outputs and workspace are
allocated with torch on the input's device, and the C entry point of the same
name runs every step on the GPU, on torch's current stream.  There is no CPU
path: importing this package fails if the library has not been built.

    score_full(...)          full-vocabulary LSE / selected logprob / entropy
    score_support_ids(...)   recorded-support logprob / entropy (+ synthetic-EOS fallback)
    score_transforms(...)    top-k / top-p / min-p support scores and descriptor
    l1_distance(...)         draft/target softmax L1 and accept_rate
"""

from __future__ import annotations

import ctypes

import torch

from . import _capi
from ._capi import (  # noqa: F401
    ROW_BAD_INPUT,
    ROW_EMPTY_SUPPORT,
    ROW_FULL_VOCAB_FALLBACK,
    ROW_SUPPORT_TRUNCATED,
    ROW_TARGET_OUTSIDE_SUPPORT,
    VsSource,
)

_LIB = None


class _Lazy:
    """Loads libvocabscore.so on first use; raises ImportError if it was never built."""

    def __getattr__(self, name):
        global _LIB
        if _LIB is None:
            _LIB = _capi.load()
        return getattr(_LIB, name)


_lib = _Lazy()

__all__ = ["score_full", "score_support_ids", "score_transforms", "l1_distance", "workspace_size",
           "status_string", "sweep_timer", "sweep_timer_ms", "VsError", "lib"]


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = _capi.load()
    return _LIB


class VsError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} (code {code})")


def status_string(code: int) -> str:
    return _lib.vs_status_string(int(code)).decode()


_DT = {torch.bfloat16: _capi.VS_BF16, torch.float32: _capi.VS_F32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_cuda(name, t, dtypes=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} dtype {t.dtype} not in {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _rowmajor(name, t):
    if t.stride(-1) != 1 or (t.dim() == 2 and t.size(0) > 1 and t.stride(0) < t.size(1)):
        raise ValueError(f"{name} must be row-major with unit inner stride")
    return t.stride(0) if t.dim() == 2 else t.size(-1)


def _make_source(logits=None, hidden=None, weight=None, temperature=1.0):
    src = VsSource()
    if logits is not None:
        _check_cuda("logits", logits, _DT, 2)
        src.kind = _capi.VS_SRC_LOGITS
        src.logits = logits.data_ptr()
        src.logits_dtype = _DT[logits.dtype]
        src.ld_logits = _rowmajor("logits", logits)
        src.T, src.V = logits.shape
        src.H = 0
        dev = logits.device
    else:
        if hidden is None or weight is None:
            raise ValueError("give either logits, or hidden and weight")
        _check_cuda("hidden", hidden, _DT, 2)
        _check_cuda("weight", weight, {torch.bfloat16}, 2)
        if hidden.size(1) != weight.size(1):
            raise ValueError("hidden and weight disagree on H")
        src.kind = _capi.VS_SRC_HIDDEN_WEIGHT
        src.hidden = hidden.data_ptr()
        src.hidden_dtype = _DT[hidden.dtype]
        src.ld_hidden = _rowmajor("hidden", hidden)
        src.weight = weight.data_ptr()
        src.weight_dtype = _capi.VS_BF16
        src.ld_weight = _rowmajor("weight", weight)
        src.T, src.H = hidden.shape
        src.V = weight.size(0)
        dev = hidden.device
    keep = None
    if isinstance(temperature, torch.Tensor):
        _check_cuda("temperature", temperature, {torch.float32}, 1)
        if temperature.numel() != src.T or not temperature.is_contiguous():
            raise ValueError("temperature must be a contiguous [T] float32 tensor")
        src.temperature = temperature.data_ptr()
        src.temperature_scalar = 1.0
        keep = temperature
    else:
        src.temperature = None
        src.temperature_scalar = float(temperature)
    return src, dev, keep


def workspace_size(op: int, src: VsSource, width: int = 0) -> int:
    return int(_lib.vs_workspace_size(op, ctypes.byref(src), int(width)))


def _workspace(op, src, dev, width=0):
    n = workspace_size(op, src, width)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev), n


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ids(name, t, T):
    _check_cuda(name, t, {torch.int64}, 1)
    if t.numel() != T or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [T] int64 tensor")


def score_full(targets, *, logits=None, hidden=None, weight=None, temperature=1.0, vocab_chunk=8192,
               with_entropy=True, with_lse=True):
    """Full-vocabulary LSE, selected logprob and entropy (vs_score_full)."""
    src, dev, _keep = _make_source(logits, hidden, weight, temperature)
    _ids("targets", targets, src.T)
    T = src.T
    lse = torch.empty(T, dtype=torch.float32, device=dev) if with_lse else None
    logprob = torch.empty(T, dtype=torch.float32, device=dev)
    entropy = torch.empty(T, dtype=torch.float32, device=dev) if with_entropy else None
    status = torch.empty(T, dtype=torch.uint8, device=dev)
    ws, n = _workspace(_capi.VS_OP_SCORE_FULL, src, dev)
    rc = _lib.vs_score_full(ctypes.byref(src), _ptr(targets), int(vocab_chunk), _ptr(lse), _ptr(logprob),
                            _ptr(entropy), _ptr(status), _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_full")
    return {"lse": lse, "logprob": logprob, "entropy": entropy, "status": status}


def score_support_ids(targets, support_ids, *, logits=None, hidden=None, weight=None, temperature=1.0,
                      fallback=None, vocab_chunk=8192, with_entropy=True):
    """Recorded-support logprob and entropy (vs_score_support_ids)."""
    src, dev, _keep = _make_source(logits, hidden, weight, temperature)
    _ids("targets", targets, src.T)
    _check_cuda("support_ids", support_ids, {torch.int64}, 2)
    if support_ids.size(0) != src.T:
        raise ValueError("support_ids must have T rows")
    width = support_ids.size(1)
    ld_ids = _rowmajor("support_ids", support_ids) if width else 0
    if fallback is not None:
        _check_cuda("fallback", fallback, {torch.uint8, torch.bool}, 1)
        if fallback.numel() != src.T or not fallback.is_contiguous():
            raise ValueError("fallback must be a contiguous [T] uint8 tensor")
        if fallback.dtype == torch.bool:
            fallback = fallback.to(torch.uint8)
    T = src.T
    logprob = torch.empty(T, dtype=torch.float32, device=dev)
    entropy = torch.empty(T, dtype=torch.float32, device=dev) if with_entropy else None
    status = torch.empty(T, dtype=torch.uint8, device=dev)
    ws, n = _workspace(_capi.VS_OP_SCORE_SUPPORT, src, dev, width)
    rc = _lib.vs_score_support_ids(ctypes.byref(src), _ptr(support_ids) if width else None, width, ld_ids,
                                   _ptr(targets), _ptr(fallback), int(vocab_chunk), _ptr(logprob), _ptr(entropy),
                                   _ptr(status), _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_support_ids")
    return {"logprob": logprob, "entropy": entropy, "status": status}


def score_transforms(targets, logits, top_k, top_p, min_p, *, temperature=1.0, cap=0, with_full_lse=True):
    """Top-k / top-p / min-p support scores and support descriptor (vs_score_transforms)."""
    src, dev, _keep = _make_source(logits=logits, temperature=temperature)
    T = src.T
    _ids("targets", targets, T)
    for name, t, dt in (("top_k", top_k, torch.int32), ("top_p", top_p, torch.float32),
                        ("min_p", min_p, torch.float32)):
        _check_cuda(name, t, {dt}, 1)
        if t.numel() != T or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T] tensor")
    out = {
        "logprob": torch.empty(T, dtype=torch.float32, device=dev),
        "entropy": torch.empty(T, dtype=torch.float32, device=dev),
        "status": torch.empty(T, dtype=torch.uint8, device=dev),
        "support_len": torch.empty(T, dtype=torch.int32, device=dev),
        "threshold_logit": torch.empty(T, dtype=torch.float32, device=dev),
        "threshold_ties": torch.empty(T, dtype=torch.int32, device=dev),
        "support_ids": torch.empty((T, cap), dtype=torch.int64, device=dev) if cap > 0 else None,
        "full_lse": torch.empty(T, dtype=torch.float32, device=dev) if with_full_lse else None,
    }
    ws, n = _workspace(_capi.VS_OP_SCORE_TRANSFORMS, src, dev)
    rc = _lib.vs_score_transforms(ctypes.byref(src), _ptr(top_k), _ptr(top_p), _ptr(min_p), _ptr(targets),
                                  _ptr(out["logprob"]), _ptr(out["entropy"]), _ptr(out["status"]),
                                  _ptr(out["support_len"]), _ptr(out["threshold_logit"]), _ptr(out["threshold_ties"]),
                                  _ptr(out["support_ids"]), int(cap), _ptr(out["full_lse"]), _ptr(ws), n,
                                  _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_transforms")
    return out


def l1_distance(target_logits, draft_logits):
    """Per-row softmax L1 distance and accept_rate (vs_l1_distance)."""
    _check_cuda("target_logits", target_logits, _DT, 2)
    _check_cuda("draft_logits", draft_logits, _DT, 2)
    if target_logits.shape != draft_logits.shape or target_logits.dtype != draft_logits.dtype:
        raise ValueError("target and draft logits must have the same shape and dtype")
    T, V = target_logits.shape
    dev = target_logits.device
    l1 = torch.empty(T, dtype=torch.float32, device=dev)
    acc = torch.empty(T, dtype=torch.float32, device=dev)
    src = VsSource()
    src.T, src.V = T, V
    ws, n = _workspace(_capi.VS_OP_L1_DISTANCE, src, dev)
    rc = _lib.vs_l1_distance(_ptr(target_logits), _ptr(draft_logits), _DT[target_logits.dtype], T, V,
                             _rowmajor("target_logits", target_logits), _rowmajor("draft_logits", draft_logits),
                             _ptr(l1), _ptr(acc), _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_l1_distance")
    return {"l1": l1, "accept_rate": acc}


def sweep_timer(enable: bool) -> None:
    """Bracket the main sweep kernel(s) of every later call with two HIP events (vs_sweep_timer)."""
    rc = _lib.vs_sweep_timer(1 if enable else 0)
    if rc:
        raise VsError(rc, "vs_sweep_timer")


def sweep_timer_ms() -> float:
    """Length of the most recent bracket, in ms; waits for it (vs_sweep_timer_ms)."""
    ms = ctypes.c_float()
    rc = _lib.vs_sweep_timer_ms(ctypes.byref(ms))
    if rc:
        raise VsError(rc, "vs_sweep_timer_ms")
    return float(ms.value)
