"""ctypes wrapper of the fp64 CPU oracle (``kd_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the library path.  It shares no code
with the HIP library.  See ``kd_oracle.c`` for the definition it implements and
the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kd_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkdoracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        i64, f64 = ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.kdo_full.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, f64, f64,
                                 vp, vp, vp, vp, vp]
        lib.kdo_full.restype = ctypes.c_int
        lib.kdo_rows.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, f64, f64,
                                 vp, vp, vp]
        lib.kdo_rows.restype = ctypes.c_int
        lib.kdo_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def num_threads() -> int:
    return int(_load().kdo_num_threads())


def full(H, W, topk_idx, topk_logit, ignore=None, tau=1.0, g=1.0, chunk=0,
         grads=True) -> dict:
    """Loss, lse, row losses and (optionally) grad_H, grad_W of the whole problem.

    ``chunk`` = rows per slice (0 = all rows at once, the dense evaluation).
    Returns fp64 arrays.
    """
    lib = _load()
    H = _f32(H)
    W = _f32(W)
    T, d = H.shape
    V = W.shape[0]
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32).reshape(T, -1)
    K = idx.shape[1]
    lg = _f32(topk_logit).reshape(T, K)
    ig = None if ignore is None else np.ascontiguousarray(ignore, dtype=np.uint8)
    loss = np.zeros(1)
    lse = np.zeros(T)
    rl = np.zeros(T)
    gH = np.zeros((T, d)) if grads else None
    gW = np.zeros((V, d)) if grads else None
    rc = lib.kdo_full(T, d, V, K, int(chunk), _ptr(H), _ptr(W), _ptr(idx), _ptr(lg), _ptr(ig),
                      float(tau), float(g), _ptr(loss), _ptr(lse), _ptr(rl), _ptr(gH), _ptr(gW))
    if rc != 0:
        raise RuntimeError(f"kdo_full failed with code {rc}")
    out = dict(loss=float(loss[0]), lse=lse, row_loss=rl)
    if grads:
        out.update(grad_H=gH, grad_W=gW)
    return out


def rows(rows_sel, H_rows, W, idx_rows, logit_rows, ignore, T, tau=1.0, g=1.0,
         grad_h=True) -> dict:
    """lse, row loss and grad_H for selected positions only (row-local quantities).

    ``ignore`` covers all T positions (it fixes N); the other per-row arrays hold
    only the selected rows, in the order of ``rows_sel``.
    """
    lib = _load()
    r = np.ascontiguousarray(rows_sel, dtype=np.int64)
    n = r.size
    Hr = _f32(H_rows).reshape(n, -1)
    d = Hr.shape[1]
    W = _f32(W)
    V = W.shape[0]
    ir = np.ascontiguousarray(idx_rows, dtype=np.int32).reshape(n, -1)
    K = ir.shape[1]
    lr = _f32(logit_rows).reshape(n, K)
    ig = None if ignore is None else np.ascontiguousarray(ignore, dtype=np.uint8)
    lse = np.zeros(n)
    rl = np.zeros(n)
    gH = np.zeros((n, d)) if grad_h else None
    rc = lib.kdo_rows(int(T), d, V, K, n, _ptr(r), _ptr(Hr), _ptr(W), _ptr(ir), _ptr(lr),
                      _ptr(ig), float(tau), float(g), _ptr(lse), _ptr(rl), _ptr(gH))
    if rc != 0:
        raise RuntimeError(f"kdo_rows failed with code {rc}")
    out = dict(lse=lse, row_loss=rl)
    if grad_h:
        out["grad_H"] = gH
    return out
