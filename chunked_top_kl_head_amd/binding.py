"""Thin ctypes binding of the C ABI in ``include/kd_topk_kl.h``.

Argument marshalling only: it checks tensor placement, allocates the outputs
and the workspace with torch (device memory plumbing) and calls the library on
the current torch stream.  Every step of the loss runs in the HIP kernels of
``libkdtopk.so``; there is no fallback path, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkdtopk.so")

KD_OK, KD_ERR_NULL, KD_ERR_SHAPE, KD_ERR_VALUE, KD_ERR_ALIGN = 0, 1, 2, 3, 4
KD_ERR_WORKSPACE, KD_ERR_UNSUPPORTED, KD_ERR_HIP, KD_ERR_INTERNAL = 5, 6, 7, 8
KD_BF16, KD_F32 = 0, 1
KD_OP_FORWARD, KD_OP_BACKWARD, KD_OP_FUSED = 0, 1, 2
KD_FLAG_ACCUMULATE_GRAD_W, KD_FLAG_LOGIT_BF16 = 1, 2

# every entry point the header declares
EXPORTS = (
    "kd_topk_kl_default_chunk",
    "kd_topk_kl_workspace_size",
    "kd_topk_kl_forward",
    "kd_topk_kl_backward",
    "kd_topk_kl_fused",
    "kd_topk_kl_fused_noalloc",
    "kd_topk_kl_validate",
    "kd_topk_kl_scale_grads",
    "kd_topk_kl_set_stage_events",
    "kd_status_string",
    "kd_topk_select",
    "kd_teacher_topk_workspace_size",
    "kd_teacher_topk",
)
KD_STAGE_LOGITS, KD_STAGE_ROWS, KD_STAGE_GRAD_H, KD_STAGE_GRAD_W = 0, 1, 2, 3
STAGE_NAMES = ("logits", "rows", "grad_H", "grad_W")


class KdProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("V", ctypes.c_int64), ("K", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32), ("temperature", ctypes.c_float),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KdSelectProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("V", ctypes.c_int64), ("K", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KdTeacherProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("V", ctypes.c_int64), ("K", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KdError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load ``libkdtopk.so`` (built by ``chunked_top_kl_head_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    prob = ctypes.POINTER(KdProblem)
    lib.kd_topk_kl_default_chunk.argtypes = [prob]
    lib.kd_topk_kl_default_chunk.restype = ctypes.c_int64
    lib.kd_topk_kl_workspace_size.argtypes = [prob, ctypes.c_int, ctypes.POINTER(sz)]
    lib.kd_topk_kl_workspace_size.restype = ctypes.c_int
    lib.kd_topk_kl_forward.argtypes = [prob, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_topk_kl_forward.restype = ctypes.c_int
    lib.kd_topk_kl_backward.argtypes = [prob, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_topk_kl_backward.restype = ctypes.c_int
    lib.kd_topk_kl_fused.argtypes = [prob, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_topk_kl_fused.restype = ctypes.c_int
    lib.kd_topk_kl_fused_noalloc.argtypes = [prob, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kd_topk_kl_fused_noalloc.restype = ctypes.c_int
    lib.kd_topk_kl_validate.argtypes = [prob, vp, vp, vp, vp, vp]
    lib.kd_topk_kl_validate.restype = ctypes.c_int
    lib.kd_topk_kl_scale_grads.argtypes = [prob, vp, vp, vp, vp, vp, ctypes.c_int32, vp]
    lib.kd_topk_kl_scale_grads.restype = ctypes.c_int
    lib.kd_topk_kl_set_stage_events.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.kd_topk_kl_set_stage_events.restype = ctypes.c_int
    lib.kd_topk_select.argtypes = [ctypes.POINTER(KdSelectProblem), vp, vp, vp, vp]
    lib.kd_topk_select.restype = ctypes.c_int
    lib.kd_teacher_topk_workspace_size.argtypes = [ctypes.POINTER(KdTeacherProblem), ctypes.POINTER(sz)]
    lib.kd_teacher_topk_workspace_size.restype = ctypes.c_int
    lib.kd_teacher_topk.argtypes = [ctypes.POINTER(KdTeacherProblem), vp, vp, vp, vp, vp, sz, vp]
    lib.kd_teacher_topk.restype = ctypes.c_int
    lib.kd_status_string.argtypes = [ctypes.c_int]
    lib.kd_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kd_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != KD_OK:
        raise KdError(fn, status, status_string(status))


def problem(T: int, d: int, V: int, K: int, temperature: float = 1.0, dtype=torch.bfloat16,
            chunk: int = 0, flags: int = 0) -> KdProblem:
    if dtype == torch.bfloat16:
        dt = KD_BF16
    elif dtype == torch.float32:
        dt = KD_F32
    else:
        raise ValueError(f"unsupported dtype {dtype}")
    return KdProblem(int(T), int(d), int(V), int(K), int(chunk), dt, float(temperature), int(flags), 0)


def default_chunk(prob: KdProblem) -> int:
    return int(load_library().kd_topk_kl_default_chunk(ctypes.byref(prob)))


def workspace_size(prob: KdProblem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check("kd_topk_kl_workspace_size", load_library().kd_topk_kl_workspace_size(ctypes.byref(prob), int(op),
                                                                                 ctypes.byref(n)))
    return int(n.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _prep(H, W, topk_idx, topk_logit, ignore):
    for name, t in (("H", H), ("W", W), ("topk_idx", topk_idx), ("topk_logit", topk_logit)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if topk_idx.dtype != torch.int32 or topk_logit.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("topk_idx must be int32 and topk_logit float32 or bfloat16")
    if H.dtype != W.dtype:
        raise ValueError("H and W must share a dtype")
    if ignore is not None and (ignore.dtype != torch.uint8 or not ignore.is_cuda or not ignore.is_contiguous()):
        raise ValueError("ignore must be a contiguous uint8 device tensor")
    T, d = H.shape
    V = W.shape[0]
    K = topk_idx.shape[1] if topk_idx.dim() == 2 else 1
    return T, d, V, K


def _flags(topk_logit, accumulate=False) -> int:
    return (KD_FLAG_LOGIT_BF16 if topk_logit.dtype == torch.bfloat16 else 0) | \
        (KD_FLAG_ACCUMULATE_GRAD_W if accumulate else 0)


def _workspace(prob, op, workspace, device):
    need = workspace_size(prob, op)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    return workspace, need


def kd_topk_kl_forward(H, W, topk_idx, topk_logit, ignore=None, temperature=1.0, chunk=0,
                       want_row_loss=False, workspace=None, stream=None):
    """Returns (loss[1], lse[T], row_loss[T] or None)."""
    T, d, V, K = _prep(H, W, topk_idx, topk_logit, ignore)
    prob = problem(T, d, V, K, temperature, H.dtype, chunk, _flags(topk_logit))
    ws, _ = _workspace(prob, KD_OP_FORWARD, workspace, H.device)
    loss = torch.empty(1, dtype=torch.float32, device=H.device)
    lse = torch.empty(T, dtype=torch.float32, device=H.device)
    rl = torch.empty(T, dtype=torch.float32, device=H.device) if want_row_loss else None
    st = load_library().kd_topk_kl_forward(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit),
                                           _ptr(ignore), _ptr(loss), _ptr(lse), _ptr(rl), _ptr(ws), ws.numel(),
                                           _stream(stream))
    _check("kd_topk_kl_forward", st)
    return loss, lse, rl


def kd_topk_kl_backward(H, W, topk_idx, topk_logit, lse, ignore=None, grad_loss=None, temperature=1.0, chunk=0,
                        workspace=None, stream=None, grad_H=None, grad_W=None, accumulate=False):
    """Returns (grad_H[T, d] in H's dtype, grad_W[V, d] fp32).  accumulate: add into the given grad_W."""
    T, d, V, K = _prep(H, W, topk_idx, topk_logit, ignore)
    if accumulate and grad_W is None:
        raise ValueError("accumulate needs the grad_W to add into")
    prob = problem(T, d, V, K, temperature, H.dtype, chunk, _flags(topk_logit, accumulate))
    ws, _ = _workspace(prob, KD_OP_BACKWARD, workspace, H.device)
    gH = torch.empty_like(H) if grad_H is None else grad_H
    gW = torch.empty((V, d), dtype=torch.float32, device=H.device) if grad_W is None else grad_W
    st = load_library().kd_topk_kl_backward(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit),
                                            _ptr(ignore), _ptr(lse), _ptr(grad_loss), _ptr(gH), _ptr(gW), _ptr(ws),
                                            ws.numel(), _stream(stream))
    _check("kd_topk_kl_backward", st)
    return gH, gW


def kd_topk_kl_fused(H, W, topk_idx, topk_logit, ignore=None, grad_loss=None, temperature=1.0, chunk=0,
                     want_lse=False, want_row_loss=False, workspace=None, stream=None, grad_H=None, grad_W=None,
                     loss=None, accumulate=False):
    """Returns (loss[1], grad_H, grad_W, lse or None, row_loss or None).  accumulate: add into the given grad_W."""
    T, d, V, K = _prep(H, W, topk_idx, topk_logit, ignore)
    if accumulate and grad_W is None:
        raise ValueError("accumulate needs the grad_W to add into")
    prob = problem(T, d, V, K, temperature, H.dtype, chunk, _flags(topk_logit, accumulate))
    ws, _ = _workspace(prob, KD_OP_FUSED, workspace, H.device)
    loss = torch.empty(1, dtype=torch.float32, device=H.device) if loss is None else loss
    lse = torch.empty(T, dtype=torch.float32, device=H.device) if want_lse else None
    rl = torch.empty(T, dtype=torch.float32, device=H.device) if want_row_loss else None
    gH = torch.empty_like(H) if grad_H is None else grad_H
    gW = torch.empty((V, d), dtype=torch.float32, device=H.device) if grad_W is None else grad_W
    st = load_library().kd_topk_kl_fused(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit),
                                         _ptr(ignore), _ptr(grad_loss), _ptr(loss), _ptr(lse), _ptr(rl), _ptr(gH),
                                         _ptr(gW), _ptr(ws), ws.numel(), _stream(stream))
    _check("kd_topk_kl_fused", st)
    return loss, gH, gW, lse, rl


def kd_topk_kl_fused_noalloc(H, W, topk_idx, topk_logit, ignore=None, *, loss, grad_H, grad_W, grad_loss=None,
                             lse=None, row_loss=None, temperature=1.0, chunk=0, accumulate=False, stream=None):
    """The fused entry on the library's static scratch: the caller passes every
    output (loss[1], grad_H [T, d], grad_W [V, d] fp32, optional lse and
    row_loss [T]); nothing is allocated here or in the library."""
    T, d, V, K = _prep(H, W, topk_idx, topk_logit, ignore)
    prob = problem(T, d, V, K, temperature, H.dtype, chunk, _flags(topk_logit, accumulate))
    st = load_library().kd_topk_kl_fused_noalloc(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(topk_idx),
                                                 _ptr(topk_logit), _ptr(ignore), _ptr(grad_loss), _ptr(loss),
                                                 _ptr(lse), _ptr(row_loss), _ptr(grad_H), _ptr(grad_W),
                                                 _stream(stream))
    _check("kd_topk_kl_fused_noalloc", st)
    return loss, grad_H, grad_W, lse, row_loss


def kd_topk_kl_validate(topk_idx, topk_logit, V, ignore=None, stream=None) -> torch.Tensor:
    """Device int64[1]: ids outside [0, V) plus kept rows without a finite teacher logit."""
    T, K = topk_idx.shape
    prob = problem(T, 8, V, K, 1.0, torch.bfloat16, 0, _flags(topk_logit))
    bad = torch.empty(1, dtype=torch.int64, device=topk_idx.device)
    st = load_library().kd_topk_kl_validate(ctypes.byref(prob), _ptr(topk_idx), _ptr(topk_logit), _ptr(ignore),
                                            _ptr(bad), _stream(stream))
    _check("kd_topk_kl_validate", st)
    return bad


def kd_topk_kl_scale_grads(grad_loss=None, grad_H=None, grad_W=None, out_H=None, out_W=None, stream=None):
    """out_H = g * grad_H and out_W = g * grad_W with g = grad_loss[0] (None: 1).

    grad_H / grad_W as returned by kd_topk_kl_fused (grad_W fp32).  An output
    left as None is the input itself (in place); out_W may be bfloat16 (the
    scaled fp32 gradient rounded to nearest even).  Returns (out_H, out_W)."""
    if grad_H is None and grad_W is None:
        return None, None
    if grad_H is not None and out_H is None:
        out_H = grad_H
    if grad_W is not None and out_W is None:
        out_W = grad_W
    for name, t in (("grad_H", grad_H), ("grad_W", grad_W), ("out_H", out_H), ("out_W", out_W)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if grad_W is not None and (grad_W.dtype != torch.float32 or out_W.shape != grad_W.shape):
        raise ValueError("grad_W must be float32 and out_W of its shape")
    if grad_H is not None and (out_H.dtype != grad_H.dtype or out_H.shape != grad_H.shape):
        raise ValueError("out_H must match grad_H")
    T, d = (grad_H.shape if grad_H is not None else (0, grad_W.shape[1]))
    V = grad_W.shape[0] if grad_W is not None else 1
    dt = grad_H.dtype if grad_H is not None else torch.bfloat16
    if out_W is None or out_W.dtype == torch.float32:
        wdt = KD_F32
    elif out_W.dtype == torch.bfloat16:
        wdt = KD_BF16
    else:
        raise ValueError(f"unsupported out_W dtype {out_W.dtype}")
    prob = problem(T, d, V, 1, 1.0, dt, 0)
    if grad_loss is not None and (grad_loss.dtype != torch.float32 or not grad_loss.is_cuda):
        raise ValueError("grad_loss must be a float32 device tensor")
    st = load_library().kd_topk_kl_scale_grads(ctypes.byref(prob), _ptr(grad_loss), _ptr(grad_H), _ptr(grad_W),
                                               _ptr(out_H), _ptr(out_W), wdt, _stream(stream))
    _check("kd_topk_kl_scale_grads", st)
    return out_H, out_W


def kd_topk_select(logits, K: int, V: Optional[int] = None, stream=None):
    """Per row of logits [T, ld] (bf16 or fp32, device), the K largest of the first V values:
    returns (topk_idx int32 [T, K], topk_logit fp32 [T, K]), descending, equal values by id."""
    if not logits.is_cuda or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D device tensor with unit column stride")
    if logits.dtype == torch.bfloat16:
        dt = KD_BF16
    elif logits.dtype == torch.float32:
        dt = KD_F32
    else:
        raise ValueError(f"unsupported dtype {logits.dtype}")
    T, n = logits.shape
    V = n if V is None else int(V)
    prob = KdSelectProblem(int(T), V, int(K), int(logits.stride(0)), dt, 0)
    idx = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    val = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    st = load_library().kd_topk_select(ctypes.byref(prob), _ptr(logits), _ptr(idx), _ptr(val), _stream(stream))
    _check("kd_topk_select", st)
    return idx, val


def kd_teacher_topk(H, W, K: int, chunk: int = 0, workspace=None, stream=None):
    """The teacher cache from hidden states H [T, d] and the lm_head W [V, d] (bf16 or fp32, device):
    per position the K largest logits H W^T and their ids, descending, equal values by id.
    Returns (topk_idx int32 [T, K], topk_logit fp32 [T, K])."""
    if not (H.is_cuda and W.is_cuda) or H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H [T, d] and W [V, d] must be device tensors with the same d")
    if H.dtype != W.dtype:
        raise ValueError("H and W must have the same dtype")
    if H.dtype == torch.bfloat16:
        dt = KD_BF16
    elif H.dtype == torch.float32:
        dt = KD_F32
    else:
        raise ValueError(f"unsupported dtype {H.dtype}")
    H, W = H.contiguous(), W.contiguous()
    T, d = H.shape
    V = W.shape[0]
    prob = KdTeacherProblem(int(T), int(d), int(V), int(K), int(chunk), dt, 0)
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check("kd_teacher_topk_workspace_size", lib.kd_teacher_topk_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=H.device)
    elif workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    idx = torch.empty((T, K), dtype=torch.int32, device=H.device)
    val = torch.empty((T, K), dtype=torch.float32, device=H.device)
    st = lib.kd_teacher_topk(ctypes.byref(prob), _ptr(H), _ptr(W), _ptr(idx), _ptr(val), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check("kd_teacher_topk", st)
    return idx, val
