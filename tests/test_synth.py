"""Checks of the seeded synthetic input generator (CPU)."""
import numpy as np
import pytest
from scipy.stats import chi2

from chunked_top_kl_head_amd import synth


def test_deterministic_under_seed():
    a = synth.make_inputs(64, 16, 500, 10, seed=5, mask=("random", 0.1))
    b = synth.make_inputs(64, 16, 500, 10, seed=5, mask=("random", 0.1))
    c = synth.make_inputs(64, 16, 500, 10, seed=6, mask=("random", 0.1))
    for f in ("H", "W", "topk_idx", "topk_logit", "ignore"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert not np.array_equal(a.topk_idx, c.topk_idx)


def test_ids_distinct_in_range_and_logits_sorted():
    x = synth.make_inputs(300, 8, 1000, 40, seed=1)
    assert x.topk_idx.dtype == np.int32 and x.topk_idx.min() >= 0 and x.topk_idx.max() < 1000
    for r in x.topk_idx:
        assert len(np.unique(r)) == 40
    assert np.all(np.diff(x.topk_logit, axis=1) <= 0)


def test_zipf_first_draw_marginal():
    """The first id of each row is a plain Zipf(1.1) draw: chi-square on the head ranks."""
    V, T = 2000, 20000
    x = synth.make_inputs(T, 8, V, 4, seed=2)
    w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    w /= w.sum()
    head = 20
    obs = np.bincount(np.minimum(x.topk_idx[:, 0], head), minlength=head + 1)
    exp = np.concatenate([w[:head], [w[head:].sum()]]) * T
    stat = ((obs - exp) ** 2 / exp).sum()
    assert stat < chi2.ppf(0.999, head)


def test_masks_exact_counts():
    x = synth.make_inputs(8192, 8, 300, 5, seed=1, mask=("random", 0.05))
    assert int(x.ignore.sum()) == 409 and x.N == 8192 - 409
    y = synth.make_inputs(4 * 512, 8, 300, 5, seed=3, mask=("trailing", 0.1, 512))
    v = y.ignore.reshape(4, 512)
    assert np.all(v[:, 512 - 51:] == 1) and np.all(v[:, :512 - 51] == 0)


def test_bf16_rounding_is_rne_and_exact():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.14159], dtype=np.float32)
    b = synth.f32_to_bf16_bits(v)
    back = synth.bf16_bits_to_f32(b)
    # ties to even: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0 + 2 ** -6)
    assert back[3] == -2.5
    x = synth.make_inputs(16, 32, 64, 4, dtype="bf16", seed=0)
    assert np.array_equal(synth.bf16_bits_to_f32(x.H_bits).reshape(x.H.shape), x.H)
    assert np.all((x.W.view(np.uint32) & 0xFFFF) == 0)


@pytest.mark.parametrize("name", ["tiny"])
def test_standard_workload_shapes(name):
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(name)
    assert x.H.shape == (w.T, w.d) and x.W.shape == (w.V, w.d)
    assert x.topk_idx.shape == (w.T, w.K) and x.ignore.shape == (w.T,)
