"""Vocabulary-scale LM-head scoring on MI355X: thin Python binding of libvocabscore.so.

Argument marshalling only: tensors are checked, outputs and workspace are
allocated with torch on the input's device, and the C entry point of the same
name runs every step on the GPU, on torch's current stream.  There is no CPU
path: importing this package fails if the library has not been built.

    score_full(...)          full-vocabulary LSE / selected logprob / entropy
    score_full_backward(...) their gradients w.r.t. the hidden state and the LM-head weight
    score_support_ids(...)   recorded-support logprob / entropy (+ synthetic-EOS fallback)
    score_transforms(...)    top-k / top-p / min-p support scores and descriptor
    sample_transforms(...)   seeded Gumbel draw from the top-k / top-p / min-p support
    l1_distance(...)         draft/target softmax L1 and accept_rate
    l1_loss(...)             weighted L1 distillation loss and its draft-logit gradient
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

__all__ = ["score_full", "score_full_backward", "score_full_noalloc", "noalloc_scratch_bytes", "score_support_ids",
           "score_support_backward",
           "score_transforms", "sample_transforms", "l1_distance", "l1_loss", "workspace_size",
           "workspace_bytes", "status_string", "sweep_timer", "sweep_timer_ms", "VsError", "lib"]


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


def _workspace(op, src, dev, width=0, given=None):
    """The call's workspace: the caller's uint8 tensor when given (checked for
    size), else a new one."""
    n = workspace_size(op, src, width)
    if given is not None:
        _check_cuda("workspace", given, {torch.uint8}, 1)
        if given.numel() < n or not given.is_contiguous():
            raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {n} bytes")
        return given, given.numel()
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev), n


def _outputs(spec, dev, out):
    """Output tensors: the caller's (``out``, a dict, checked against
    ``spec`` = {name: (shape, dtype) or None}) or new ones."""
    res = {}
    for name, sd in spec.items():
        if sd is None:
            res[name] = None
            continue
        shape, dtype = sd
        t = None if out is None else out.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
        else:
            _check_cuda(f"out[{name!r}]", t, {dtype})
            if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
                raise ValueError(f"out[{name!r}] must be a contiguous {dtype} tensor of shape {tuple(shape)}")
        res[name] = t
    return res


def workspace_bytes(op: str, *, logits=None, hidden=None, weight=None, width: int = 0) -> int:
    """Bytes of workspace an entry point needs for these inputs (vs_workspace_size);
    op is one of "score_full", "score_support_ids", "score_transforms", "l1_distance",
    "sample_transforms", "l1_loss", "score_full_backward", "score_support_backward" (width =
    the support width, or the backward's vocab_chunk)."""
    ops = {"score_full": _capi.VS_OP_SCORE_FULL, "score_support_ids": _capi.VS_OP_SCORE_SUPPORT,
           "score_transforms": _capi.VS_OP_SCORE_TRANSFORMS, "l1_distance": _capi.VS_OP_L1_DISTANCE,
           "sample_transforms": _capi.VS_OP_SAMPLE_TRANSFORMS, "l1_loss": _capi.VS_OP_L1_LOSS,
           "score_full_backward": _capi.VS_OP_SCORE_FULL_BACKWARD,
           "score_support_backward": _capi.VS_OP_SCORE_SUPPORT_BACKWARD}
    src, _, _ = _make_source(logits, hidden, weight, 1.0)
    return workspace_size(ops[op], src, width)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ids(name, t, T):
    _check_cuda(name, t, {torch.int64}, 1)
    if t.numel() != T or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [T] int64 tensor")


def score_full(targets, *, logits=None, hidden=None, weight=None, temperature=1.0, vocab_chunk=8192,
               with_entropy=True, with_lse=True, out=None, workspace=None):
    """Full-vocabulary LSE, selected logprob and entropy (vs_score_full).

    ``out`` (dict of preallocated outputs) and ``workspace`` (uint8 tensor of
    at least workspace_bytes("score_full", ...) bytes) are optional: with
    both, the call allocates nothing."""
    src, dev, _keep = _make_source(logits, hidden, weight, temperature)
    _ids("targets", targets, src.T)
    T = src.T
    o = _outputs({"lse": ((T,), torch.float32) if with_lse else None, "logprob": ((T,), torch.float32),
                  "entropy": ((T,), torch.float32) if with_entropy else None, "status": ((T,), torch.uint8)},
                 dev, out)
    ws, n = _workspace(_capi.VS_OP_SCORE_FULL, src, dev, given=workspace)
    rc = _lib.vs_score_full(ctypes.byref(src), _ptr(targets), int(vocab_chunk), _ptr(o["lse"]), _ptr(o["logprob"]),
                            _ptr(o["entropy"]), _ptr(o["status"]), _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_full")
    return o


def score_full_backward(targets, lse, entropy=None, *, hidden, weight, grad_logprob=None, grad_entropy=None,
                        temperature=1.0, vocab_chunk=8192, want_hidden=True, want_weight=True, out=None,
                        workspace=None):
    """Gradients of sum_t (grad_logprob[t] logprob_t + grad_entropy[t] entropy_t)
    with respect to the hidden state and the LM-head weight
    (vs_score_full_backward); lse / entropy are the forward's outputs.
    Returns ``grad_hidden`` [T, H] and ``grad_weight`` [V, H] (fp32)."""
    src, dev, _keep = _make_source(None, hidden, weight, temperature)
    _ids("targets", targets, src.T)
    T, H, V = src.T, src.H, src.V
    for name, t in (("lse", lse), ("entropy", entropy), ("grad_logprob", grad_logprob),
                    ("grad_entropy", grad_entropy)):
        if t is not None:
            _check_cuda(name, t, {torch.float32}, 1)
            if t.numel() != T or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [T] float32 tensor")
    o = _outputs({"grad_hidden": ((T, H), torch.float32) if want_hidden else None,
                  "grad_weight": ((V, H), torch.float32) if want_weight else None}, dev, out)
    ws, n = _workspace(_capi.VS_OP_SCORE_FULL_BACKWARD, src, dev, int(vocab_chunk), given=workspace)
    rc = _lib.vs_score_full_backward(ctypes.byref(src), _ptr(targets), _ptr(lse), _ptr(entropy), _ptr(grad_logprob),
                                     _ptr(grad_entropy), int(vocab_chunk), _ptr(o["grad_hidden"]), H,
                                     _ptr(o["grad_weight"]), H, _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_full_backward")
    return o


def score_support_backward(targets, support_ids, *, hidden, weight, grad_logprob=None, grad_entropy=None,
                           temperature=1.0, want_hidden=True, want_weight=True, out=None, workspace=None):
    """Gradients of sum_t (grad_logprob[t] logprob_t + grad_entropy[t] entropy_t)
    of the recorded-support scores (score_support_ids) with respect to the
    hidden state and the LM-head weight (vs_score_support_backward).  Returns
    ``grad_hidden`` [T, H] and ``grad_weight`` [V, H] (fp32)."""
    src, dev, _keep = _make_source(None, hidden, weight, temperature)
    T, H, V = src.T, src.H, src.V
    _ids("targets", targets, T)
    _check_cuda("support_ids", support_ids, {torch.int64}, 2)
    if support_ids.size(0) != T:
        raise ValueError("support_ids must have T rows")
    width = support_ids.size(1)
    ld_ids = _rowmajor("support_ids", support_ids) if width > 0 else 0
    for name, t in (("grad_logprob", grad_logprob), ("grad_entropy", grad_entropy)):
        if t is not None:
            _check_cuda(name, t, {torch.float32}, 1)
            if t.numel() != T or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [T] float32 tensor")
    o = _outputs({"grad_hidden": ((T, H), torch.float32) if want_hidden else None,
                  "grad_weight": ((V, H), torch.float32) if want_weight else None}, dev, out)
    ws, n = _workspace(_capi.VS_OP_SCORE_SUPPORT_BACKWARD, src, dev, int(width), given=workspace)
    rc = _lib.vs_score_support_backward(ctypes.byref(src), _ptr(support_ids) if width else None, int(width),
                                        int(ld_ids), _ptr(targets),
                                        _ptr(grad_logprob), _ptr(grad_entropy), _ptr(o["grad_hidden"]), H,
                                        _ptr(o["grad_weight"]), H, _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_support_backward")
    return o


def score_full_noalloc(targets, *, logits=None, hidden=None, weight=None, temperature=1.0, vocab_chunk=8192,
                       with_entropy=True, with_lse=True, out=None):
    """score_full through vs_score_full_noalloc: no workspace; the library's
    per-GPU scratch array serves the hidden/weight source (calls that overlap
    on one GPU race on it).  With ``out`` the call allocates nothing."""
    src, dev, _keep = _make_source(logits, hidden, weight, temperature)
    _ids("targets", targets, src.T)
    T = src.T
    o = _outputs({"lse": ((T,), torch.float32) if with_lse else None, "logprob": ((T,), torch.float32),
                  "entropy": ((T,), torch.float32) if with_entropy else None, "status": ((T,), torch.uint8)},
                 dev, out)
    rc = _lib.vs_score_full_noalloc(ctypes.byref(src), _ptr(targets), int(vocab_chunk), _ptr(o["lse"]),
                                    _ptr(o["logprob"]), _ptr(o["entropy"]), _ptr(o["status"]), _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_full_noalloc")
    return o


def noalloc_scratch_bytes() -> int:
    """Size of the per-GPU scratch array of score_full_noalloc (vs_noalloc_scratch_bytes)."""
    return int(_lib.vs_noalloc_scratch_bytes())


def score_support_ids(targets, support_ids, *, logits=None, hidden=None, weight=None, temperature=1.0,
                      fallback=None, vocab_chunk=8192, with_entropy=True, out=None, workspace=None):
    """Recorded-support logprob and entropy (vs_score_support_ids); ``out`` and
    ``workspace`` as for score_full."""
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
    o = _outputs({"logprob": ((T,), torch.float32), "entropy": ((T,), torch.float32) if with_entropy else None,
                  "status": ((T,), torch.uint8)}, dev, out)
    ws, n = _workspace(_capi.VS_OP_SCORE_SUPPORT, src, dev, width, given=workspace)
    rc = _lib.vs_score_support_ids(ctypes.byref(src), _ptr(support_ids) if width else None, width, ld_ids,
                                   _ptr(targets), _ptr(fallback), int(vocab_chunk), _ptr(o["logprob"]),
                                   _ptr(o["entropy"]), _ptr(o["status"]), _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_support_ids")
    return o


def score_transforms(targets, logits, top_k, top_p, min_p, *, hidden=None, weight=None, temperature=1.0, cap=0,
                     with_full_lse=True, out=None, workspace=None):
    """Top-k / top-p / min-p support scores and support descriptor
    (vs_score_transforms) over bf16 ``logits``, or (``logits=None``) over the
    bf16-rounded projection of ``hidden`` and ``weight``; ``out`` and
    ``workspace`` as for score_full."""
    src, dev, _keep = _make_source(logits, hidden, weight, temperature)
    T = src.T
    _ids("targets", targets, T)
    for name, t, dt in (("top_k", top_k, torch.int32), ("top_p", top_p, torch.float32),
                        ("min_p", min_p, torch.float32)):
        _check_cuda(name, t, {dt}, 1)
        if t.numel() != T or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T] tensor")
    out = _outputs({
        "logprob": ((T,), torch.float32),
        "entropy": ((T,), torch.float32),
        "status": ((T,), torch.uint8),
        "support_len": ((T,), torch.int32),
        "threshold_logit": ((T,), torch.float32),
        "threshold_ties": ((T,), torch.int32),
        "support_ids": ((T, cap), torch.int64) if cap > 0 else None,
        "full_lse": ((T,), torch.float32) if with_full_lse else None,
    }, dev, out)
    ws, n = _workspace(_capi.VS_OP_SCORE_TRANSFORMS, src, dev, given=workspace)
    rc = _lib.vs_score_transforms(ctypes.byref(src), _ptr(top_k), _ptr(top_p), _ptr(min_p), _ptr(targets),
                                  _ptr(out["logprob"]), _ptr(out["entropy"]), _ptr(out["status"]),
                                  _ptr(out["support_len"]), _ptr(out["threshold_logit"]), _ptr(out["threshold_ties"]),
                                  _ptr(out["support_ids"]), int(cap), _ptr(out["full_lse"]), _ptr(ws), n,
                                  _stream(dev))
    if rc:
        raise VsError(rc, "vs_score_transforms")
    return out


def sample_transforms(logits, top_k, top_p, min_p, *, seed, offset=0, hidden=None, weight=None, temperature=1.0,
                      out=None, workspace=None):
    """Seeded Gumbel draw of one token per row from the top-k / top-p / min-p
    support (vs_sample_transforms), over bf16 ``logits`` or (``logits=None``)
    the bf16-rounded projection of ``hidden`` and ``weight``.  Returns
    ``sampled`` (int64, -1 on a BAD_INPUT row), ``status`` and the support
    descriptor; ``out`` and ``workspace`` as for score_full."""
    src, dev, _keep = _make_source(logits, hidden, weight, temperature)
    T = src.T
    for name, t, dt in (("top_k", top_k, torch.int32), ("top_p", top_p, torch.float32),
                        ("min_p", min_p, torch.float32)):
        _check_cuda(name, t, {dt}, 1)
        if t.numel() != T or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T] tensor")
    o = _outputs({"sampled": ((T,), torch.int64), "status": ((T,), torch.uint8),
                  "support_len": ((T,), torch.int32), "threshold_logit": ((T,), torch.float32),
                  "threshold_ties": ((T,), torch.int32)}, dev, out)
    ws, n = _workspace(_capi.VS_OP_SAMPLE_TRANSFORMS, src, dev, given=workspace)
    rc = _lib.vs_sample_transforms(ctypes.byref(src), _ptr(top_k), _ptr(top_p), _ptr(min_p),
                                   int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1), _ptr(o["sampled"]),
                                   _ptr(o["status"]), _ptr(o["support_len"]), _ptr(o["threshold_logit"]),
                                   _ptr(o["threshold_ties"]), _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_sample_transforms")
    return o


def l1_distance(target_logits, draft_logits, *, out=None):
    """Per-row softmax L1 distance and accept_rate (vs_l1_distance); ``out`` as
    for score_full (this call needs no workspace)."""
    _check_cuda("target_logits", target_logits, _DT, 2)
    _check_cuda("draft_logits", draft_logits, _DT, 2)
    if target_logits.shape != draft_logits.shape or target_logits.dtype != draft_logits.dtype:
        raise ValueError("target and draft logits must have the same shape and dtype")
    T, V = target_logits.shape
    dev = target_logits.device
    o = _outputs({"l1": ((T,), torch.float32), "accept_rate": ((T,), torch.float32)}, dev, out)
    src = VsSource()
    src.T, src.V = T, V
    n = workspace_size(_capi.VS_OP_L1_DISTANCE, src, 0)
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    rc = _lib.vs_l1_distance(_ptr(target_logits), _ptr(draft_logits), _DT[target_logits.dtype], T, V,
                             _rowmajor("target_logits", target_logits), _rowmajor("draft_logits", draft_logits),
                             _ptr(o["l1"]), _ptr(o["accept_rate"]), _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_l1_distance")
    return o


def l1_loss(target_logits, draft_logits, *, weights=None, grad_scale=1.0, with_grad=True, grad_dtype=None,
            out=None, workspace=None):
    """Weighted L1 distillation loss and its draft-logit gradient (vs_l1_loss).

    Returns ``l1``, ``accept_rate``, ``loss`` (a [3] tensor: num, den,
    num / den) and ``grad`` (the gradient of grad_scale * loss with respect to
    the draft logits, in ``grad_dtype``, default the logits' dtype)."""
    _check_cuda("target_logits", target_logits, _DT, 2)
    _check_cuda("draft_logits", draft_logits, _DT, 2)
    if target_logits.shape != draft_logits.shape or target_logits.dtype != draft_logits.dtype:
        raise ValueError("target and draft logits must have the same shape and dtype")
    T, V = target_logits.shape
    dev = target_logits.device
    if weights is not None:
        _check_cuda("weights", weights, {torch.float32}, 1)
        if weights.numel() != T or not weights.is_contiguous():
            raise ValueError("weights must be a contiguous [T] float32 tensor")
    gdt = grad_dtype or draft_logits.dtype
    o = _outputs({"l1": ((T,), torch.float32), "accept_rate": ((T,), torch.float32), "loss": ((3,), torch.float32),
                  "grad": ((T, V), gdt) if with_grad else None}, dev, out)
    src = VsSource()
    src.T, src.V = T, V
    ws, n = _workspace(_capi.VS_OP_L1_LOSS, src, dev, given=workspace)
    rc = _lib.vs_l1_loss(_ptr(target_logits), _ptr(draft_logits), _DT[target_logits.dtype], T, V,
                         _rowmajor("target_logits", target_logits), _rowmajor("draft_logits", draft_logits),
                         _ptr(weights), float(grad_scale), _ptr(o["l1"]), _ptr(o["accept_rate"]), _ptr(o["loss"]),
                         _ptr(o["grad"]), _DT[gdt], V if with_grad else 0, _ptr(ws), n, _stream(dev))
    if rc:
        raise VsError(rc, "vs_l1_loss")
    return o


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
