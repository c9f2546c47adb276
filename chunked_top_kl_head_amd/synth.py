"""Seeded synthetic inputs for the fused top-K KL distillation loss.

This module only draws inputs; it contains none of the loss arithmetic, so
both the fp64 oracle (under ``oracle/``) and the HIP path can consume the same
arrays without sharing any method code.

What is drawn, per position t (the pages' workloads, with synthetic values in
place of the corpora, caches and weights that are not available here):

* ``H[T, d]``  student hidden states, i.i.d. N(0, 1).
* ``W[V, d]``  student output projection (lm_head), i.i.d. N(0, 0.02^2).
* ``topk_idx[T, K]``  K *distinct* teacher token ids, drawn i.i.d. from a
  Zipf(1.1) law over the vocabulary (weight proportional to (v+1)^-1.1, token
  ids taken to be in frequency order) and de-duplicated in draw order.  The
  offline teacher cache keeps the top-100 tokens per position
  (ai-thai.com/posts/846, Thai translation of "Efficient Knowledge
  Distillation for LLMs: Offline Top-K Logits and a Fused Chunked KL Loss",
  section "Offline distillation").
* ``topk_logit[T, K]``  the teacher's cached logits: K draws of
  3 * Gumbel(0, 1) sorted in descending order, so the first id drawn gets the
  largest logit (a cache ranked by teacher probability).
* ``ignore[T]`` uint8, non-zero = position excluded from the loss.

bf16 inputs are drawn in fp32 and rounded to bfloat16 with round-to-nearest-
even; the arrays returned hold the exact rounded values (as fp32 views and as
raw 16-bit patterns) so that every consumer sees bit-identical operands.

Seeds: workload i of the standard list uses ``SeedSequence(20261203 + i)``
spawned into five independent streams [H, W, idx, logit, mask].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 20261203
ZIPF_EXPONENT = 1.1
GUMBEL_SCALE = 3.0
W_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic workload."""

    name: str
    T: int
    d: int
    V: int
    K: int
    tau: float
    dtype: str            # "bf16" or "f32"
    chunk: int            # chunk rows C used by the library on this workload
    mask: Optional[tuple] = None   # None | ("random", frac) | ("trailing", frac, seq_len)
    seed_index: int = 0

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of one fused fwd+bwd step: three T*d*V GEMMs."""
        return 6.0 * self.T * self.d * self.V


# The five standard workloads (shapes of the pages' experiments: gpt-oss
# vocabulary 201,088, top-100 cache, 8K-256K positions).
WORKLOADS = {
    "tiny": Workload("tiny", T=256, d=256, V=4096, K=16, tau=1.0, dtype="f32",
                     chunk=64, mask=None, seed_index=0),
    "llama3b": Workload("llama3b", T=8192, d=3072, V=128256, K=100, tau=1.0,
                        dtype="bf16", chunk=1024, mask=("random", 0.05), seed_index=1),
    "gptoss20b": Workload("gptoss20b", T=32768, d=2880, V=201088, K=100, tau=1.0,
                          dtype="bf16", chunk=8192, mask=None, seed_index=2),
    "batched4x32k": Workload("batched4x32k", T=131072, d=2880, V=201088, K=100, tau=2.0,
                             dtype="bf16", chunk=8192, mask=("trailing", 0.1, 32768),
                             seed_index=3),
    "extreme256k": Workload("extreme256k", T=262144, d=2880, V=201088, K=100, tau=1.0,
                            dtype="bf16", chunk=8192, mask=None, seed_index=4),
}


# ----------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs are finite by construction.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Teacher cache draws
# ----------------------------------------------------------------------------
def _zipf_cdf(V: int) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-ZIPF_EXPONENT)
    c = np.cumsum(w)
    return c / c[-1]


def _distinct_zipf_ids(rng: np.random.Generator, rows: int, V: int, K: int,
                       block: int = 8192) -> np.ndarray:
    """K distinct ids per row: i.i.d. Zipf draws, repeats discarded, draw order kept.

    This has the law of successive sampling without replacement.  Rows are
    processed in fixed blocks so the random stream consumption, and therefore
    the result, is a pure function of (seed, rows, V, K).
    """
    if K > V:
        raise ValueError("K > V")
    cdf = _zipf_cdf(V)
    out = np.empty((rows, K), dtype=np.int32)
    first = max(2 * K, 64)
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        n = r1 - r0
        draws = np.searchsorted(cdf, rng.random((n, first)), side="right").astype(np.int32)
        np.minimum(draws, V - 1, out=draws)
        pending = np.arange(n)
        while True:
            d = draws[pending]
            order = np.argsort(d, axis=1, kind="stable")
            srt = np.take_along_axis(d, order, axis=1)
            dup_s = np.zeros(srt.shape, dtype=bool)
            dup_s[:, 1:] = srt[:, 1:] == srt[:, :-1]
            dup = np.empty_like(dup_s)
            np.put_along_axis(dup, order, dup_s, axis=1)
            keep = ~dup
            cnt = np.cumsum(keep, axis=1)
            ok = cnt[:, -1] >= K
            if ok.any():
                sel = keep[ok] & (cnt[ok] <= K)
                out[r0 + pending[ok]] = d[ok][sel].reshape(-1, K)
            if ok.all():
                break
            pending = pending[~ok]
            more = np.searchsorted(cdf, rng.random((pending.size, first)), side="right").astype(np.int32)
            np.minimum(more, V - 1, out=more)
            # rows that need more draws get them appended (still draw order)
            grown = np.concatenate([draws[pending], more], axis=1)
            draws = np.zeros((n, grown.shape[1]), dtype=np.int32)
            draws[pending] = grown
    return out


def _teacher_logits(rng: np.random.Generator, rows: int, K: int) -> np.ndarray:
    g = rng.gumbel(0.0, 1.0, size=(rows, K)) * GUMBEL_SCALE
    g = -np.sort(-g, axis=1)               # descending: rank 0 = largest
    return np.ascontiguousarray(g, dtype=np.float32)


# ----------------------------------------------------------------------------
# Public API
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Inputs:
    T: int
    d: int
    V: int
    K: int
    tau: float
    dtype: str
    H: np.ndarray           # fp32 [T, d], exact values of the operand (bf16-rounded if dtype=bf16)
    W: np.ndarray           # fp32 [V, d], likewise
    topk_idx: np.ndarray    # int32 [T, K]
    topk_logit: np.ndarray  # fp32 [T, K]
    ignore: np.ndarray      # uint8 [T]
    H_bits: Optional[np.ndarray] = None   # uint16 [T, d] when dtype=bf16
    W_bits: Optional[np.ndarray] = None   # uint16 [V, d] when dtype=bf16

    @property
    def N(self) -> int:
        return int((self.ignore == 0).sum())


def make_inputs(T: int, d: int, V: int, K: int, *, tau: float = 1.0, dtype: str = "bf16",
                seed: int = 0, mask: Optional[tuple] = None,
                h_std: float = 1.0, w_std: float = W_STD) -> Inputs:
    """Draw one seeded problem.  ``seed`` selects ``SeedSequence(SEED_BASE + seed)``."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    ss = np.random.SeedSequence(SEED_BASE + seed).spawn(5)
    rH, rW, rI, rL, rM = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    H = rH.standard_normal((T, d), dtype=np.float32)
    if h_std != 1.0:
        H *= np.float32(h_std)
    W = rW.standard_normal((V, d), dtype=np.float32)
    W *= np.float32(w_std)
    idx = _distinct_zipf_ids(rI, T, V, K) if T > 0 else np.zeros((0, K), np.int32)
    logit = _teacher_logits(rL, T, K)
    ignore = np.zeros(T, dtype=np.uint8)
    if mask is not None and T > 0:
        kind = mask[0]
        if kind == "random":
            n = int(np.floor(mask[1] * T))
            ignore[rM.choice(T, size=n, replace=False)] = 1
        elif kind == "trailing":
            frac, seq = mask[1], mask[2]
            if T % seq:
                raise ValueError("trailing mask needs T to be a multiple of the sequence length")
            pad = int(np.floor(frac * seq))
            view = ignore.reshape(-1, seq)
            if pad:
                view[:, seq - pad:] = 1
        elif kind == "all":
            ignore[:] = 1
        else:
            raise ValueError(kind)
    Hb = Wb = None
    if dtype == "bf16":
        Hb = f32_to_bf16_bits(H)
        Wb = f32_to_bf16_bits(W)
        H = bf16_bits_to_f32(Hb).reshape(T, d)
        W = bf16_bits_to_f32(Wb).reshape(V, d)
    return Inputs(T=T, d=d, V=V, K=K, tau=float(tau), dtype=dtype, H=H, W=W,
                  topk_idx=idx, topk_logit=logit, ignore=ignore, H_bits=Hb, W_bits=Wb)


def workload_inputs(name: str) -> Inputs:
    """Inputs of one standard workload (see ``WORKLOADS``)."""
    w = WORKLOADS[name]
    return make_inputs(w.T, w.d, w.V, w.K, tau=w.tau, dtype=w.dtype,
                       seed=w.seed_index, mask=w.mask)
