"""Thin ctypes binding of libfldce.so (the C ABI in include/fldce.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory (inputs, outputs, workspace) and the
current HIP stream.  If the library is missing the first call raises; there is
no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FLDCE_LIB may point at another build of the same library (A/B timing)
LIB_PATH = os.environ.get("FLDCE_LIB") or os.path.join(_HERE, "libfldce.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
REDUCTION_SUM, REDUCTION_MEAN = 0, 1

_c_int, _c_i64, _c_f, _c_p, _c_sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes); every function the header declares
_SIGNATURES = {
    "fldce_version": (_c_int, []),
    "fldce_status_string": (ctypes.c_char_p, [_c_int]),
    "fldce_default_chunk_rows": (_c_i64, [_c_i64, _c_i64, _c_i64]),
    "fldce_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int, _c_i64]),
    "fldce_fwd_bwd": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_i64,
                               _c_f, _c_f, _c_int, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                               _c_p, _c_sz, _c_p]),
    "fldce_fwd_bwd_ex": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int,
                                  _c_i64, _c_f, _c_f, _c_int, _c_i64, _c_i64, _c_f, _c_p, _c_p,
                                  _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_sz, _c_p]),
    "fldce_fwd_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int]),
    "fldce_fwd": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_i64,
                           _c_f, _c_f, _c_int, _c_i64, _c_i64, _c_f, _c_p, _c_p, _c_p, _c_p, _c_sz,
                           _c_p]),
    "fldce_fwd_noalloc": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int,
                                   _c_i64, _c_f, _c_f, _c_int, _c_i64, _c_i64, _c_f, _c_p, _c_p,
                                   _c_p, _c_p]),
    "fldce_scale_grads": (_c_int, [_c_p, _c_int, _c_p, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_p]),
    "fldce_shard_partials_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int]),
    "fldce_shard_partials": (_c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_int,
                                      _c_i64, _c_f, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "fldce_shard_bwd_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int, _c_i64]),
    "fldce_shard_bwd": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64,
                                 _c_i64, _c_int, _c_i64, _c_f, _c_f, _c_int, _c_i64, _c_p, _c_p,
                                 _c_i64, _c_p, _c_sz, _c_p]),
    "fldce_profile_num_stages": (_c_int, []),
    "fldce_profile_stage_name": (ctypes.c_char_p, [_c_int]),
    "fldce_profile_begin": (_c_int, []),
    "fldce_profile_end": (_c_int, []),
    "fldce_profile_read": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


class FldceError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfldce.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name, None)
            if f is None:  # an older build (FLDCE_LIB): calling it raises AttributeError
                continue
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fldce_status_string(status).decode()


def fldce_version() -> int:
    return lib().fldce_version()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return DTYPE_F32
    if t == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t}")


def _reduction_code(r) -> int:
    if r in ("sum", REDUCTION_SUM):
        return REDUCTION_SUM
    if r in ("mean", REDUCTION_MEAN):
        return REDUCTION_MEAN
    raise ValueError(f"reduction must be 'mean' or 'sum', got {r!r}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t: torch.Tensor, name: str, dtype=None, device=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_inputs(h, W, target, p_mask=None, bias=None, lse=None, w_name="W"):
    """Size, device, layout and dtype checks of the inputs (the kernels read
    exactly N rows of h, target, p_mask and lse and V rows of W and bias):
    returns (N, H, V).  Sizes are checked first."""
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError(f"h and {w_name} must be 2-D, got {tuple(h.shape)} and {tuple(W.shape)}")
    N, H = h.shape
    V = W.shape[0]
    if W.shape[1] != H:
        raise ValueError(f"{w_name} must have {H} columns like h, got {W.shape[1]}")
    for name, t, n in (("target", target, N), ("p_mask", p_mask, N), ("lse", lse, N),
                       ("bias", bias, V)):
        if t is not None and t.numel() != n:
            raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")
    _check(h, "h")
    d = h.device
    _check(W, w_name, h.dtype, d)
    _check(target, "target", torch.int64, d)
    for name, t in (("p_mask", p_mask), ("lse", lse)):
        if t is not None:
            _check(t, name, torch.float32, d)
    if bias is not None:
        _check(bias, "bias", h.dtype, d)
    return N, H, V

def _out(out: Optional[dict], name: str, numel: int, like: torch.Tensor, dtype=None,
         shape=None) -> torch.Tensor:
    """The caller's output tensor ``out[name]`` (checked: device, contiguous,
    dtype and element count, so no kernel writes past it) or a new one of
    ``shape`` (default: like ``like``)."""
    dtype = like.dtype if dtype is None else dtype
    t = (out or {}).get(name)
    if t is None:
        if shape is None:
            return torch.empty_like(like, dtype=dtype)
        return torch.empty(shape, dtype=dtype, device=like.device)
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    _check(t, name, dtype, like.device)
    return t


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _workspace(nbytes: int, dev, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        _check(ws, "workspace", None, dev)
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)


def fldce_profile_begin() -> None:
    lib().fldce_profile_begin()


def fldce_profile_end() -> None:
    lib().fldce_profile_end()


def fldce_profile_num_stages() -> int:
    return lib().fldce_profile_num_stages()


def fldce_profile_stage_name(stage: int) -> str:
    return lib().fldce_profile_stage_name(stage).decode()


def fldce_profile_read(stage: int):
    """(total_ms, launches) of a stage since fldce_profile_begin (after a sync)."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    rc = lib().fldce_profile_read(stage, ctypes.byref(ms), ctypes.byref(n))
    if rc != 0:
        raise FldceError(rc, "fldce_profile_read")
    return ms.value, n.value


def fldce_default_chunk_rows(N: int, H: int, V: int) -> int:
    return lib().fldce_default_chunk_rows(N, H, V)


def fldce_workspace_size(N: int, H: int, V: int, dtype, chunk_rows: int = 0) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return lib().fldce_workspace_size(N, H, V, code, chunk_rows)


def fldce_shard_partials_workspace_size(N: int, H: int, V_local: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return lib().fldce_shard_partials_workspace_size(N, H, V_local, code)


def fldce_shard_bwd_workspace_size(N: int, H: int, V_local: int, dtype, chunk_rows: int = 0) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return lib().fldce_shard_bwd_workspace_size(N, H, V_local, code, chunk_rows)


def fldce_fwd_bwd(h: torch.Tensor, W: torch.Tensor, target: torch.Tensor,
                  p_mask: Optional[torch.Tensor] = None, ignore_index: int = -100,
                  label_smoothing: float = 0.0, logit_scale: float = 1.0,
                  reduction="mean", total: int = 0, chunk_rows: int = 0,
                  row_stats: bool = False, workspace: Optional[torch.Tensor] = None,
                  out: Optional[dict] = None) -> dict:
    """loss, dH, dW (and per-row lse / loss with row_stats) of the fused LM-head
    cross-entropy.  h [N,H], W [V,H] (fp32 or bf16, same dtype), target int64
    [N], p_mask fp32 [N] or None.  Outputs may be passed in ``out``."""
    N, H, V = _check_inputs(h, W, target, p_mask)
    dev = h.device
    code = _dtype_code(h.dtype)
    loss = _out(out, "loss", 1, h, torch.float32, (1,))
    dH = _out(out, "dH", N * H, h)
    dW = _out(out, "dW", V * H, W)
    lse = rl = None
    if row_stats:
        lse = _out(out, "row_lse", N, h, torch.float32, (N,))
        rl = _out(out, "row_loss", N, h, torch.float32, (N,))
    nbytes = lib().fldce_workspace_size(N, H, V, code, chunk_rows)
    ws = _workspace(nbytes, dev, workspace)
    with torch.cuda.device(dev):
        rc = lib().fldce_fwd_bwd(_ptr(h), _ptr(W), _ptr(target), _ptr(p_mask), N, H, V, code,
                                 ignore_index, label_smoothing, logit_scale,
                                 _reduction_code(reduction), total, _ptr(loss), _ptr(dH), _ptr(dW),
                                 _ptr(lse), _ptr(rl), chunk_rows, _ptr(ws), nbytes, _stream(dev))
    if rc != 0:
        raise FldceError(rc, "fldce_fwd_bwd")
    r = dict(loss=loss, dH=dH, dW=dW)
    if row_stats:
        r.update(row_lse=lse, row_loss=rl)
    return r


def _eob_code(eob_token_id: Optional[int]) -> int:
    return -1 if eob_token_id is None else int(eob_token_id)


def fldce_fwd_bwd_ex(h: torch.Tensor, W: torch.Tensor, target: torch.Tensor,
                     p_mask: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                     ignore_index: int = -100, label_smoothing: float = 0.0,
                     logit_scale: float = 1.0, reduction="mean", total: int = 0,
                     eob_token_id: Optional[int] = None, eob_weight: float = 1.0,
                     want_db: Optional[bool] = None, chunk_rows: int = 0,
                     row_stats: bool = False, workspace: Optional[torch.Tensor] = None,
                     out: Optional[dict] = None, want_dH: bool = True,
                     want_dW: bool = True) -> dict:
    """fldce_fwd_bwd plus page 1's optional bias [V] (and its gradient db,
    returned when ``want_db`` or, by default, when a bias is given) and the
    end-of-block weight (rows whose target is ``eob_token_id``).  With
    ``want_dH`` / ``want_dW`` False that gradient is not computed (None).
    Outputs may be passed in ``out`` (loss, dH, dW, db, row_lse, row_loss)."""
    N, H, V = _check_inputs(h, W, target, p_mask, bias)
    dev = h.device
    code = _dtype_code(h.dtype)
    want_db = (bias is not None) if want_db is None else want_db
    loss = _out(out, "loss", 1, h, torch.float32, (1,))
    dH = _out(out, "dH", N * H, h) if want_dH else None
    dW = _out(out, "dW", V * H, W) if want_dW else None
    db = _out(out, "db", V, h, h.dtype, (V,)) if want_db else None
    lse = rl = None
    if row_stats:
        lse = _out(out, "row_lse", N, h, torch.float32, (N,))
        rl = _out(out, "row_loss", N, h, torch.float32, (N,))
    nbytes = lib().fldce_workspace_size(N, H, V, code, chunk_rows)
    ws = _workspace(nbytes, dev, workspace)
    with torch.cuda.device(dev):
        rc = lib().fldce_fwd_bwd_ex(_ptr(h), _ptr(W), _ptr(bias), _ptr(target), _ptr(p_mask), N, H, V,
                                    code, ignore_index, label_smoothing, logit_scale,
                                    _reduction_code(reduction), total, _eob_code(eob_token_id),
                                    eob_weight, _ptr(loss), _ptr(dH), _ptr(dW), _ptr(db), _ptr(lse),
                                    _ptr(rl), chunk_rows, _ptr(ws), nbytes, _stream(dev))
    if rc != 0:
        raise FldceError(rc, "fldce_fwd_bwd_ex")
    r = dict(loss=loss, dH=dH, dW=dW, db=db)
    if row_stats:
        r.update(row_lse=lse, row_loss=rl)
    return r


def fldce_fwd_workspace_size(N: int, H: int, V: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return lib().fldce_fwd_workspace_size(N, H, V, code)


def fldce_fwd(h: torch.Tensor, W: torch.Tensor, target: torch.Tensor,
              p_mask: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
              ignore_index: int = -100, label_smoothing: float = 0.0, logit_scale: float = 1.0,
              reduction="mean", total: int = 0, eob_token_id: Optional[int] = None,
              eob_weight: float = 1.0, row_stats: bool = False,
              workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None) -> dict:
    """Forward only: loss (and per-row lse / loss with row_stats), no gradients.
    Outputs may be passed in ``out`` (loss, row_lse, row_loss)."""
    N, H, V = _check_inputs(h, W, target, p_mask, bias)
    dev = h.device
    code = _dtype_code(h.dtype)
    loss = _out(out, "loss", 1, h, torch.float32, (1,))
    lse = rl = None
    if row_stats:
        lse = _out(out, "row_lse", N, h, torch.float32, (N,))
        rl = _out(out, "row_loss", N, h, torch.float32, (N,))
    nbytes = lib().fldce_fwd_workspace_size(N, H, V, code)
    ws = _workspace(nbytes, dev, workspace)
    with torch.cuda.device(dev):
        rc = lib().fldce_fwd(_ptr(h), _ptr(W), _ptr(bias), _ptr(target), _ptr(p_mask), N, H, V, code,
                             ignore_index, label_smoothing, logit_scale, _reduction_code(reduction),
                             total, _eob_code(eob_token_id), eob_weight, _ptr(loss), _ptr(lse),
                             _ptr(rl), _ptr(ws), nbytes, _stream(dev))
    if rc != 0:
        raise FldceError(rc, "fldce_fwd")
    r = dict(loss=loss)
    if row_stats:
        r.update(row_lse=lse, row_loss=rl)
    return r


# bytes of the library's own device array that fldce_fwd_noalloc uses
NOALLOC_SCRATCH_BYTES = 64 << 20


def fldce_fwd_noalloc(h: torch.Tensor, W: torch.Tensor, target: torch.Tensor,
                      p_mask: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                      ignore_index: int = -100, label_smoothing: float = 0.0,
                      logit_scale: float = 1.0, reduction="mean", total: int = 0,
                      eob_token_id: Optional[int] = None, eob_weight: float = 1.0,
                      row_stats: bool = False, out: Optional[dict] = None) -> dict:
    """fldce_fwd without a workspace: the library's own per-device array
    (NOALLOC_SCRATCH_BYTES) holds the intermediates.  The caller passes every
    output in ``out`` (loss, and row_lse / row_loss with row_stats) so that
    nothing is allocated; missing ones are created here (convenience only)."""
    N, H, V = _check_inputs(h, W, target, p_mask, bias)
    dev = h.device
    code = _dtype_code(h.dtype)
    loss = _out(out, "loss", 1, h, torch.float32, (1,))
    lse = rl = None
    if row_stats:
        lse = _out(out, "row_lse", N, h, torch.float32, (N,))
        rl = _out(out, "row_loss", N, h, torch.float32, (N,))
    with torch.cuda.device(dev):
        rc = lib().fldce_fwd_noalloc(_ptr(h), _ptr(W), _ptr(bias), _ptr(target), _ptr(p_mask), N,
                                     H, V, code, ignore_index, label_smoothing, logit_scale,
                                     _reduction_code(reduction), total, _eob_code(eob_token_id),
                                     eob_weight, _ptr(loss), _ptr(lse), _ptr(rl), _stream(dev))
    if rc != 0:
        raise FldceError(rc, "fldce_fwd_noalloc")
    r = dict(loss=loss)
    if row_stats:
        r.update(row_lse=lse, row_loss=rl)
    return r


def fldce_scale_grads(grad_out: torch.Tensor, dH: Optional[torch.Tensor] = None,
                      dW: Optional[torch.Tensor] = None, db: Optional[torch.Tensor] = None) -> None:
    """In place: each given gradient *= grad_out (a float32 device scalar),
    skipped on the device when grad_out == 1."""
    _check(grad_out, "grad_out", torch.float32)
    if grad_out.numel() != 1:
        raise ValueError("grad_out must hold one element")
    ts = [t for t in (dH, dW, db) if t is not None]
    if not ts:
        return
    dtype = ts[0].dtype
    for name, t in (("dH", dH), ("dW", dW), ("db", db)):
        if t is not None:
            _check(t, name, dtype, grad_out.device)
    n = lambda t: 0 if t is None else t.numel()  # noqa: E731
    with torch.cuda.device(grad_out.device):
        rc = lib().fldce_scale_grads(_ptr(grad_out), _dtype_code(dtype), _ptr(dH), n(dH), _ptr(dW),
                                     n(dW), _ptr(db), n(db), _stream(grad_out.device))
    if rc != 0:
        raise FldceError(rc, "fldce_scale_grads")


def fldce_shard_partials(h: torch.Tensor, W_local: torch.Tensor, target: torch.Tensor,
                         vocab_start: int, ignore_index: int = -100, logit_scale: float = 1.0,
                         sumlogit: bool = True, workspace: Optional[torch.Tensor] = None,
                         out: Optional[dict] = None) -> dict:
    """Per-row (max, sum-exp, target logit, sum of logits) of one vocabulary
    shard.  Outputs may be passed in ``out`` (row_max, row_sumexp,
    target_logit, row_sumlogit)."""
    N, H, V_local = _check_inputs(h, W_local, target, w_name="W_local")
    dev = h.device
    code = _dtype_code(h.dtype)
    f = lambda name: _out(out, name, N, h, torch.float32, (N,))  # noqa: E731
    m, S, t = f("row_max"), f("row_sumexp"), f("target_logit")
    r = f("row_sumlogit") if sumlogit else None
    nbytes = lib().fldce_shard_partials_workspace_size(N, H, V_local, code)
    ws = _workspace(nbytes, dev, workspace)
    with torch.cuda.device(dev):
        rc = lib().fldce_shard_partials(_ptr(h), _ptr(W_local), _ptr(target), N, H, V_local,
                                        vocab_start, code, ignore_index, logit_scale, _ptr(m),
                                        _ptr(S), _ptr(t), _ptr(r), _ptr(ws), nbytes, _stream(dev))
    if rc != 0:
        raise FldceError(rc, "fldce_shard_partials")
    return dict(row_max=m, row_sumexp=S, target_logit=t, row_sumlogit=r)


def fldce_shard_bwd(h: torch.Tensor, W_local: torch.Tensor, target: torch.Tensor,
                    p_mask: Optional[torch.Tensor], lse: torch.Tensor, vocab_start: int,
                    V_global: int, ignore_index: int = -100, label_smoothing: float = 0.0,
                    logit_scale: float = 1.0, reduction="mean", total: int = 0,
                    chunk_rows: int = 0, workspace: Optional[torch.Tensor] = None,
                    out: Optional[dict] = None) -> dict:
    """dH_partial (fp32) and dW_local of one vocabulary shard given the global
    lse.  Outputs may be passed in ``out`` (dH_partial, dW_local)."""
    N, H, V_local = _check_inputs(h, W_local, target, p_mask, lse=lse, w_name="W_local")
    dev = h.device
    code = _dtype_code(h.dtype)
    dHp = _out(out, "dH_partial", N * H, h, torch.float32, (N, H))
    dWl = _out(out, "dW_local", V_local * H, W_local)
    nbytes = lib().fldce_shard_bwd_workspace_size(N, H, V_local, code, chunk_rows)
    ws = _workspace(nbytes, dev, workspace)
    with torch.cuda.device(dev):
        rc = lib().fldce_shard_bwd(_ptr(h), _ptr(W_local), _ptr(target), _ptr(p_mask), _ptr(lse), N,
                                   H, V_local, vocab_start, V_global, code, ignore_index,
                                   label_smoothing, logit_scale, _reduction_code(reduction), total,
                                   _ptr(dHp), _ptr(dWl), chunk_rows, _ptr(ws), nbytes, _stream(dev))
    if rc != 0:
        raise FldceError(rc, "fldce_shard_bwd")
    return dict(dH_partial=dHp, dW_local=dWl)
