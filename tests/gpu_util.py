"""Helpers of the GPU parity tests: device upload and the comparison bars."""
from __future__ import annotations

import numpy as np
import torch

# Parity bar for bf16 operands with fp32 accumulation:
#   loss: relative error <= 1e-3; grad_H, grad_W: max-abs error <= 2e-2 * max|ref|.
BF16_TOL = dict(loss=1e-3, grad=2e-2, lse=1e-4, row=1e-3)
# fp32 operands: fp32 MFMA, fp32 G, hardware exp2/log2 (about 1 ulp)
F32_TOL = dict(loss=1e-5, grad=1e-4, lse=1e-5, row=1e-5)


def tol_for(dtype: str) -> dict:
    return BF16_TOL if dtype == "bf16" else F32_TOL


def upload(x, device="cuda"):
    """Device tensors of a synth.Inputs problem (bf16 operands from the exact bits)."""
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).to(device).view(torch.bfloat16)
        W = torch.from_numpy(x.W_bits.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        H = torch.from_numpy(x.H).to(device)
        W = torch.from_numpy(x.W).to(device)
    idx = torch.from_numpy(x.topk_idx).to(device)
    lg = torch.from_numpy(x.topk_logit).to(device)
    ig = torch.from_numpy(x.ignore).to(device) if x.ignore.any() else None
    return dict(H=H.contiguous(), W=W.contiguous(), topk_idx=idx.contiguous(), topk_logit=lg.contiguous(),
                ignore=ig)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def rel_maxabs(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(a - ref))) if ref.size else 0.0
    if scale == 0.0:
        return err
    return err / scale


def loss_rel(a: float, ref: float) -> float:
    return abs(a - ref) / max(abs(ref), 1e-30) if ref != 0 else abs(a)
