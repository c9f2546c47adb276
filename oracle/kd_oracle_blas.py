"""fp64 CPU oracle of the fused top-K KL loss, with library matrix products.

TEST INFRASTRUCTURE ONLY: imported by the tests (never by the library path).
It shares no code with the HIP library, nor with ``kd_oracle.c``: it is a
second, independent writing of the same definition, fast enough for the
full-vocabulary workloads (a chunk of 8,192 positions against a 201,088-token
vocabulary, or the Llama-3B-like workload in full) that the plain C loops of
``kd_oracle.c`` cannot finish in test time.

Definition (the plain reading of the pages; they fix no formula).  Pages:
[TH] ai-thai.com/posts/846, Thai translation of the Hugging Face post
"Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
Chunked KL Loss", section "Fused Chunked KL Loss", items "Dense KL" (the
teacher distribution is rebuilt from the cached top-100 logits) and "Fused
chunked KL" (per slice of positions: project the hidden states to logits,
fold them into the loss, drop them); [PT] ai2day.live/pt, "O que os
investigadores alteraram?" (the loss measures how far the student's
predictions are from the teacher's).

    a_tv  = (H_t . W_v) / tau               lse_t = log sum_v exp(a_tv)
    p_tk  = softmax_k(l_tk / tau)           (0 where l_tk = -inf)
    L_t   = sum_{k: p_tk > 0} p_tk (log p_tk - a_{t, idx_tk} + lse_t)
    loss  = (1/N) sum_{t kept} L_t          (0 when N = 0)
    G_tv  = g / (tau N) (exp(a_tv - lse_t) sum_k p_tk - P_tv),  P_tv = sum_{k: idx_tk = v} p_tk
    grad_H = G W,  grad_W = G^T H           (G = 0 on ignored rows)

Per chunk of C rows the steps are taken in that order, in plain PyTorch CPU
float64 ops (multithreaded): the three contractions (the student logits
H_c W^T, G W and G^T H_c) are library matrix products, the student softmax
is exp(a - max) divided by its sum, and the cached entries of G are
scattered with accumulation (duplicates add up).  Inputs are fp32 arrays
holding exact operand values (bf16 widens exactly); outputs are numpy fp64.
"""
from __future__ import annotations

import numpy as np
import torch

F64 = torch.float64


def _teacher(logit_rows: torch.Tensor, tau: float):
    """p and log p of the teacher over the cached entries of some rows ([TH] "Dense KL")."""
    b = logit_rows.to(F64) / tau
    M = b.amax(dim=1, keepdim=True)
    if not bool(torch.isfinite(M).all()):
        raise ValueError("a kept position has no finite teacher logit")
    logS = torch.log(torch.exp(b - M).sum(dim=1, keepdim=True))
    logp = b - M - logS
    p = torch.exp(logp)                  # exactly 0 where the logit is -inf
    return p, logp


def full(H, W, topk_idx, topk_logit, ignore=None, tau=1.0, g=1.0, chunk=0, grads=True, w_rows=None) -> dict:
    """Loss, lse[T], row losses[T] and, with ``grads``, grad_H[T, d] and grad_W[V, d] (fp64).

    ``chunk`` = rows per slice (0: all rows at once, the dense evaluation).
    ``w_rows``: compute grad_W only at these vocabulary rows (returned as
    ``grad_W_rows`` [len(w_rows), d]; grad_H and the full grad_W are skipped).
    """
    H32 = torch.from_numpy(np.ascontiguousarray(H, dtype=np.float32))
    T, d = H32.shape
    W64 = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).to(F64)
    V = W64.shape[0]
    idx = torch.from_numpy(np.ascontiguousarray(topk_idx).reshape(T, -1).astype(np.int64))
    K = idx.shape[1]
    lg = torch.from_numpy(np.ascontiguousarray(topk_logit, dtype=np.float32).reshape(T, K))
    kept = (torch.ones(T, dtype=torch.bool) if ignore is None
            else torch.from_numpy(np.ascontiguousarray(ignore).reshape(T) == 0))
    N = int(kept.sum())
    s = g / (tau * N) if N > 0 else 0.0
    C = T if chunk <= 0 or chunk >= T else int(chunk)
    sel = None if w_rows is None else torch.from_numpy(np.asarray(w_rows, dtype=np.int64))

    lse = torch.zeros(T, dtype=F64)
    row_loss = torch.zeros(T, dtype=F64)
    gH = torch.zeros((T, d), dtype=F64) if grads and sel is None else None
    gW = torch.zeros((V, d), dtype=F64) if grads and sel is None else None
    gWr = torch.zeros((sel.numel(), d), dtype=F64) if grads and sel is not None else None
    for t0 in range(0, T, C):
        t1 = min(T, t0 + C)
        Hc = H32[t0:t1].to(F64)
        # student logits of the slice over the full vocabulary, their
        # logsumexp, and the softmax numerators exp(a - max)
        a = Hc @ W64.T
        a /= tau
        m = a.amax(dim=1)
        E = torch.exp(a - m[:, None])
        S = E.sum(dim=1)
        l_c = m + torch.log(S)
        lse[t0:t1] = l_c
        rows = torch.nonzero(kept[t0:t1]).reshape(-1)      # kept rows of the slice (local)
        if rows.numel() == 0:
            continue
        p, logp = _teacher(lg[t0 + rows], tau)
        ids = idx[t0 + rows]
        a_at = a[rows[:, None], ids]
        pos = p > 0.0
        terms = torch.where(pos, p * (torch.where(pos, logp, torch.zeros_like(logp)) - a_at + l_c[rows, None]),
                            torch.zeros_like(p))
        row_loss[t0 + rows] = terms.sum(dim=1)
        if not grads:
            continue
        psum = p.sum(dim=1)
        rows_rep = rows.repeat_interleave(K)
        if sel is None:
            # G of the slice: s (q psum - P), zero on ignored rows; q = E / S
            G = torch.zeros_like(a)
            G[rows] = E[rows] / S[rows, None] * (s * psum[:, None])
            G.index_put_((rows_rep, ids.reshape(-1)), -s * p.reshape(-1), accumulate=True)
            gH[t0:t1] = G @ W64
            gW += G.T @ Hc
        else:
            Gs = torch.zeros((t1 - t0, sel.numel()), dtype=F64)
            Gs[rows] = E[rows][:, sel] / S[rows, None] * (s * psum[:, None])
            # cached entries that fall on a selected row
            where = torch.full((V,), -1, dtype=torch.int64)
            where[sel] = torch.arange(sel.numel())
            hit = where[ids]
            rr, kk = torch.nonzero(hit >= 0, as_tuple=True)
            Gs.index_put_((rows[rr], hit[rr, kk]), -s * p[rr, kk], accumulate=True)
            gWr += Gs.T @ Hc
        del a, E
    loss = float(row_loss[kept].sum() / N) if N > 0 else 0.0
    out = dict(loss=loss, lse=lse.numpy(), row_loss=row_loss.numpy())
    if grads and sel is None:
        out.update(grad_H=gH.numpy(), grad_W=gW.numpy())
    elif grads:
        out["grad_W_rows"] = gWr.numpy()
    return out


def rows(rows_sel, H_rows, W, idx_rows, logit_rows, ignore, T, tau=1.0, g=1.0, grad_h=True) -> dict:
    """lse, row loss and grad_H of selected positions (row-local quantities; N from ignore[T])."""
    r = np.asarray(rows_sel, dtype=np.int64)
    ig = np.zeros(T, np.uint8) if ignore is None else np.asarray(ignore, dtype=np.uint8)
    n = r.size
    kept_all = int((ig == 0).sum())
    # evaluate the selected rows as a problem of their own, then restore N
    sub_ignore = ig[r]
    res = full(np.asarray(H_rows).reshape(n, -1), W, idx_rows, logit_rows, sub_ignore, tau=tau, g=1.0,
               grads=grad_h)
    out = dict(lse=res["lse"], row_loss=res["row_loss"])
    if grad_h:
        n_sub = int((sub_ignore == 0).sum())
        # G scales with g / (tau N): rescale from the sub-problem's N to the full one
        out["grad_H"] = res["grad_H"] * (g * n_sub / kept_all if kept_all > 0 else 0.0)
    return out
