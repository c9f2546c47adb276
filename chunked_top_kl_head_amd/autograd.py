"""torch.autograd integration of the fused chunked top-K KL loss.

``topk_kl_loss`` is the loss of ``include/kd_topk_kl.h`` as a differentiable
function of the student's hidden states H and output projection W, for use
inside a training step ([TH] ai-thai.com/posts/846, section "Fused Chunked KL
Loss", item "Fused chunked KL": the projection is fused into the loss, so the
caller hands over hidden states and the weight instead of logits).

Two modes, both running every step of the loss in the HIP library:

* ``"fused"`` (default): the forward runs ``kd_topk_kl_fused`` with g = 1 and
  keeps the gradients; the backward writes them, scaled by the upstream
  gradient, into fresh tensors with ``kd_topk_kl_scale_grads`` (grad_W in the
  weight's dtype), so a retained graph can be differentiated again.  Three
  contractions per chunk.
* ``"recompute"``: the forward runs ``kd_topk_kl_forward`` and keeps only lse
  [T]; the backward runs ``kd_topk_kl_backward`` with the upstream gradient,
  recomputing each chunk's logits (the pages' backward).  Four contractions
  per chunk, no [T, d] + [V, d] gradient held between forward and backward.

When neither H nor W requires a gradient, the forward runs
``kd_topk_kl_forward`` only and keeps nothing.  Leading dimensions of H
(batch, sequence) are flattened; topk_idx may be int64 (as ``torch.topk``
returns it) and is converted to int32; topk_logit may be float32 or bfloat16.
No gradient flows to the teacher cache.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B


class TopKKLLossFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, topk_idx, topk_logit, ignore, temperature, chunk, mode):
        if mode not in ("fused", "recompute"):
            raise ValueError(f"unknown mode {mode!r}")
        lead = H.shape[:-1]
        d = H.shape[-1]
        H2 = H.reshape(-1, d).contiguous()
        idx = topk_idx.reshape(H2.shape[0], -1)
        idx = (idx if idx.dtype == torch.int32 else idx.to(torch.int32)).contiguous()
        logit = topk_logit.reshape(H2.shape[0], -1).contiguous()
        ign = None if ignore is None else ignore.reshape(-1).to(torch.uint8).contiguous()
        W2 = W.contiguous()
        ctx.lead, ctx.temperature, ctx.chunk = lead, float(temperature), int(chunk)
        ctx.w_dtype = W.dtype
        ctx.need = (bool(ctx.needs_input_grad[0]), bool(ctx.needs_input_grad[1]))
        if not any(ctx.need):
            # no gradient wanted: the loss alone, nothing kept
            ctx.mode = "none"
            loss, _, _ = B.kd_topk_kl_forward(H2, W2, idx, logit, ign, temperature=temperature, chunk=chunk)
            return loss.reshape(())
        ctx.mode = mode
        if mode == "fused":
            loss, gH, gW, _, _ = B.kd_topk_kl_fused(H2, W2, idx, logit, ign, temperature=temperature, chunk=chunk)
            ctx.save_for_backward(gH if ctx.need[0] else None, gW if ctx.need[1] else None)
        else:
            loss, lse, _ = B.kd_topk_kl_forward(H2, W2, idx, logit, ign, temperature=temperature, chunk=chunk)
            ctx.save_for_backward(H2, W2, idx, logit, lse, ign if ign is not None else torch.empty(0))
            ctx.has_ignore = ign is not None
        return loss.reshape(())

    @staticmethod
    def backward(ctx, grad_out):
        if ctx.mode == "none":
            return (None,) * 8
        need_h, need_w = ctx.need
        g = grad_out.reshape(1).to(torch.float32).contiguous()
        if ctx.mode == "fused":
            # fresh outputs: the kept gradients stay as they are, so a retained
            # graph can be differentiated again with another upstream gradient
            gH_k, gW_k = ctx.saved_tensors
            gH = torch.empty_like(gH_k) if need_h else None
            gW = torch.empty(gW_k.shape, dtype=ctx.w_dtype, device=gW_k.device) if need_w else None
            B.kd_topk_kl_scale_grads(g, gH_k if need_h else None, gW_k if need_w else None, out_H=gH, out_W=gW)
        else:
            H2, W2, idx, logit, lse, ign = ctx.saved_tensors
            gH, gW32 = B.kd_topk_kl_backward(H2, W2, idx, logit, lse, ign if ctx.has_ignore else None, grad_loss=g,
                                             temperature=ctx.temperature, chunk=ctx.chunk)
            if not need_h:
                gH = None
            if not need_w:
                gW = None
            elif ctx.w_dtype == torch.float32:
                gW = gW32
            else:
                # the fp32 accumulator rounded to the weight's dtype by the library
                _, gW = B.kd_topk_kl_scale_grads(None, grad_W=gW32,
                                                 out_W=torch.empty(gW32.shape, dtype=ctx.w_dtype, device=gW32.device))
        if gH is not None:
            gH = gH.reshape(*ctx.lead, gH.shape[-1])
        return gH, gW, None, None, None, None, None, None


def topk_kl_loss(H: torch.Tensor, W: torch.Tensor, topk_idx: torch.Tensor, topk_logit: torch.Tensor,
                 ignore: Optional[torch.Tensor] = None, temperature: float = 1.0, chunk: int = 0,
                 mode: str = "fused") -> torch.Tensor:
    """KL(teacher top-K || student) averaged over kept positions; differentiable in H and W."""
    return TopKKLLossFunction.apply(H, W, topk_idx, topk_logit, ignore, temperature, chunk, mode)
