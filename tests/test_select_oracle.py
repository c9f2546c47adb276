"""Pins of the top-K selection oracle (oracle/topk_select.py), on the CPU.

Each pin comes from outside the oracle's own lexicographic-sort formulation:
Python's float ordering with heapq for ordinary values, hand-worked rows for
the special values, and the defining properties of a top-K selection.
"""
import heapq

import numpy as np
import pytest

from chunked_top_kl_head_amd import synth
from oracle.topk_select import topk_select


def test_matches_heapq_on_ordinary_values():
    rng = np.random.default_rng(11)
    for V, K in ((1, 1), (5, 5), (50, 7), (300, 100), (1000, 1)):
        x = (rng.standard_normal((6, V)) * 3).astype(np.float32)
        x[:, ::13] = -np.inf
        ids, vals = topk_select(x, K)
        for t in range(x.shape[0]):
            row = [float(v) for v in x[t]]
            want = heapq.nlargest(K, range(V), key=lambda v: (row[v], -v))
            assert list(ids[t]) == want
            assert np.array_equal(vals[t], x[t, want])


def test_ties_ordered_by_id():
    x = np.array([[2.0, 5.0, 2.0, 5.0, 1.0, 5.0]], dtype=np.float32)
    ids, vals = topk_select(x, 5)
    assert list(ids[0]) == [1, 3, 5, 0, 2]
    assert list(vals[0]) == [5.0, 5.0, 5.0, 2.0, 2.0]


def test_signed_zero_infinities_and_nan():
    # worked by hand: NaN below -inf, -0.0 below +0.0
    x = np.array([[np.nan, -0.0, 0.0, -np.inf, 1.0, np.inf, -0.0, 0.0]], dtype=np.float32)
    ids, vals = topk_select(x, 8)
    assert list(ids[0]) == [5, 4, 2, 7, 1, 6, 3, 0]
    assert np.signbit(vals[0, 4]) and not np.signbit(vals[0, 2])
    assert np.isnan(vals[0, 7])


def test_selection_properties_on_a_tie_heavy_workload():
    rng = np.random.default_rng(3)
    x = rng.integers(-20, 20, size=(40, 2000)).astype(np.float32) / 4      # many equal values
    K = 100
    ids, vals = topk_select(x, K)
    for t in range(x.shape[0]):
        sel = ids[t]
        assert len(set(sel.tolist())) == K                                   # distinct ids
        assert np.array_equal(vals[t], x[t, sel])                            # values belong to the ids
        assert np.all(np.diff(vals[t]) <= 0)                                 # descending
        rest = np.setdiff1d(np.arange(x.shape[1]), sel)
        assert vals[t, -1] >= x[t, rest].max()                               # nothing better left out
        # among values equal to the cut-off, the smallest ids were kept
        cut = vals[t, -1]
        kept_eq = np.sort(sel[vals[t] == cut])
        all_eq = np.nonzero(x[t] == cut)[0]
        assert np.array_equal(kept_eq, all_eq[:kept_eq.size])


def test_bf16_inputs_are_returned_exactly():
    rng = np.random.default_rng(4)
    bits = synth.f32_to_bf16_bits(rng.standard_normal((3, 500)).astype(np.float32) * 4)
    x = synth.bf16_bits_to_f32(bits).reshape(3, 500)
    ids, vals = topk_select(x, 50)
    assert np.array_equal(vals, np.take_along_axis(x, ids.astype(np.int64), axis=1))
    assert np.array_equal(synth.f32_to_bf16_bits(vals), np.take_along_axis(bits, ids.astype(np.int64), axis=1))


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        topk_select(np.zeros((1, 4), np.float32), 5)
    with pytest.raises(ValueError):
        topk_select(np.zeros((1, 4), np.float32), 0)
