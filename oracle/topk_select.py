"""Oracle of the teacher top-K cache producer: per row, the K largest logits
and their ids.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark, never by the
library path; it shares no code with the HIP library.

What is computed ([TH] ai-thai.com/posts/846, Thai translation of "Efficient
Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused Chunked KL
Loss", section "Offline distillation": the teacher is run once over the
corpus and, per position, only its 100 largest logits and their token ids are
kept).  The pages do not fix an order or a rule for equal values; the reading
taken here:

* order: logits descending; equal logits by increasing id;
* "equal" and "larger" follow the total order of the IEEE bit patterns: -0.0
  sorts below +0.0, -inf is the smallest number, NaN is below everything;
* bf16 inputs are widened exactly to fp32 for the returned logits.

The definition is written directly as a lexicographic sort (numpy), one row at
a time; nothing is blocked or reordered.
"""
from __future__ import annotations

import numpy as np


def order_key(values: np.ndarray) -> np.ndarray:
    """uint32 key whose unsigned order is the order above (fp32 values)."""
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    neg = (u >> np.uint32(31)) == 1
    key = np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint32)
    key[np.isnan(values.astype(np.float32))] = np.uint32(0)
    return key


def topk_select(logits: np.ndarray, K: int):
    """(ids int32 [T, K], values float32 [T, K]) of each row of logits [T, V] (fp32 values)."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    T, V = x.shape
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    ids = np.empty((T, K), dtype=np.int32)
    vals = np.empty((T, K), dtype=np.float32)
    col = np.arange(V, dtype=np.int64)
    for t in range(T):
        key = order_key(x[t])
        # lexsort: last key is primary -> sort by key descending, then id ascending
        order = np.lexsort((col, -key.astype(np.int64)))[:K]
        ids[t] = order
        vals[t] = x[t, order]
    return ids, vals
