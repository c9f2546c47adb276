"""Pins of the fp64 oracle against facts fixed independently of its code.

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, tau in the wrong place, a transposed operand, a wrong N) fails
at least one of them:

* hand-derived closed forms (tests/golden/hand_cases.json);
* K = V: the loss equals the ordinary full KL(p || q) from scipy;
* KL >= 0 and the Gibbs bound L_t >= -log sum_k q_{idx_k} (student from numpy);
* chunked == dense: the pages state the chunked evaluations equal the dense one
  (ai-thai.com/posts/846, "Fused Chunked KL Loss" section, the three variants
  are mathematically equivalent);
* central finite differences of the loss pin the closed-form gradient;
* self-distillation, uniform student, temperature identity, mask = deletion,
  symmetries and linearity in the upstream gradient.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import log_softmax, softmax
from scipy.stats import entropy

from chunked_top_kl_head_amd.synth import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


@pytest.fixture(scope="module", params=["c_loops", "matrix_products"])
def oracle(request):
    """Every pin holds for both writings of the definition: the plain C loops
    (oracle/kd_oracle.c) and the numpy version whose contractions are library
    matrix products (oracle/kd_oracle_blas.py, used at full-vocabulary sizes)."""
    if request.param == "c_loops":
        from oracle import kd_oracle
        kd_oracle._load()
        return kd_oracle
    from oracle import kd_oracle_blas
    return kd_oracle_blas


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def _problem(T=12, d=8, V=37, K=6, tau=1.0, seed=3, mask=None, w_std=0.5):
    return make_inputs(T, d, V, K, tau=tau, dtype="f32", seed=seed, mask=mask, w_std=w_std)


def _student_logq(x, tau):
    z = x.H.astype(np.float64) @ x.W.astype(np.float64).T
    return log_softmax(z / tau, axis=1)


# --------------------------------------------------------------------------
# hand-derived closed forms
# --------------------------------------------------------------------------
def _ev(v):
    ns = {"e": math.e, "log": math.log, "ln2": float(np.float32(math.log(2.0))), "nan": float("nan")}
    if isinstance(v, str):
        return float(eval(v, {"__builtins__": {}}, ns))  # noqa: S307 (fixture expressions)
    return float(v)


def _arr(rows):
    return np.array([[_ev(c) for c in r] for r in rows], dtype=np.float64)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_derived_cases(oracle, case):
    H = _arr(case["H"]).astype(np.float32)
    W = _arr(case["W"]).astype(np.float32)
    lg = _arr(case["topk_logit"]).astype(np.float32)
    idx = np.array(case["topk_idx"], dtype=np.int32)
    ig = np.array(case["ignore"], dtype=np.uint8)
    r = oracle.full(H, W, idx, lg, ig, tau=case["tau"])
    tol = case["tol"]
    assert abs(r["loss"] - _ev(case["loss"])) <= tol * max(1.0, abs(_ev(case["loss"])))
    np.testing.assert_allclose(r["grad_H"], _arr(case["grad_H"]), rtol=0, atol=tol)
    np.testing.assert_allclose(r["grad_W"], _arr(case["grad_W"]), rtol=0, atol=tol)


# --------------------------------------------------------------------------
# K = V: ordinary full-vocabulary KL
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tau", [1.0, 2.0, 0.7])
def test_full_cache_equals_full_kl(oracle, tau):
    T, d, V = 9, 6, 23
    x = _problem(T=T, d=d, V=V, K=4, tau=tau, seed=11)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(V) for _ in range(T)]).astype(np.int32)
    lg = (rng.standard_normal((T, V)) * 2.0).astype(np.float32)
    lg[0, :3] = -np.inf                    # zero-probability teacher entries
    r = oracle.full(x.H, x.W, idx, lg, None, tau=tau, grads=False)
    logq = _student_logq(x, tau)
    q = np.exp(logq)
    ref = []
    for t in range(T):
        p = np.zeros(V)
        p[idx[t]] = softmax(lg[t].astype(np.float64) / tau)
        ref.append(entropy(p, q[t]))       # scipy: sum p log(p/q)
    ref = np.array(ref)
    np.testing.assert_allclose(r["row_loss"], ref, rtol=1e-11, atol=1e-14)
    assert abs(r["loss"] - ref.mean()) <= 1e-11 * abs(ref.mean())
    # lse of the student against scipy's logsumexp
    z = x.H.astype(np.float64) @ x.W.astype(np.float64).T
    np.testing.assert_allclose(r["lse"], np.log(np.exp(z / tau).sum(1)), rtol=1e-12)


# --------------------------------------------------------------------------
# non-negativity and the Gibbs bound
# --------------------------------------------------------------------------
def test_kl_nonnegative_and_gibbs_bound(oracle):
    x = _problem(T=40, d=16, V=300, K=20, tau=1.0, seed=4)
    r = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0, grads=False)
    logq = _student_logq(x, 1.0)
    Q = np.exp(np.take_along_axis(logq, x.topk_idx.astype(np.int64), axis=1)).sum(1)
    assert np.all(r["row_loss"] >= 0)
    assert np.all(r["row_loss"] >= -np.log(Q) - 1e-12)


# --------------------------------------------------------------------------
# chunked == dense (the pages' equivalence of the variants)
# --------------------------------------------------------------------------
def test_chunked_equals_dense(oracle):
    T = 50
    x = _problem(T=T, d=12, V=97, K=9, tau=1.5, seed=7, mask=("random", 0.2))
    dense = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.5, chunk=0)
    for C in (1, 7, 16, T):
        r = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.5, chunk=C)
        assert abs(r["loss"] - dense["loss"]) <= 1e-12 * abs(dense["loss"])
        assert _rel(r["lse"], dense["lse"]) <= 1e-14
        assert _rel(r["grad_H"], dense["grad_H"]) <= 1e-12
        assert _rel(r["grad_W"], dense["grad_W"]) <= 1e-12


def test_rows_entry_matches_full(oracle):
    T = 30
    x = _problem(T=T, d=10, V=61, K=7, tau=1.0, seed=9, mask=("random", 0.25))
    full = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0)
    sel = np.array([0, 3, 4, 17, 29])
    r = oracle.rows(sel, x.H[sel], x.W, x.topk_idx[sel], x.topk_logit[sel], x.ignore, T, tau=1.0)
    np.testing.assert_allclose(r["lse"], full["lse"][sel], rtol=1e-14)
    np.testing.assert_allclose(r["row_loss"], full["row_loss"][sel], rtol=1e-13, atol=1e-16)
    assert _rel(r["grad_H"], full["grad_H"][sel]) <= 1e-13


# --------------------------------------------------------------------------
# finite differences
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_finite_differences(oracle, tau):
    T, d, V, K = 3, 5, 11, 4
    x = _problem(T=T, d=d, V=V, K=K, tau=tau, seed=13, w_std=0.7)
    ig = np.array([0, 1, 0], dtype=np.uint8)
    base = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, ig, tau=tau)

    def loss_at(H, W):
        return oracle.full(H, W, x.topk_idx, x.topk_logit, ig, tau=tau, grads=False)["loss"]

    h = 1e-3
    for name, arr, grad in (("H", x.H, base["grad_H"]), ("W", x.W, base["grad_W"])):
        fd = np.zeros(arr.shape)
        for i in np.ndindex(arr.shape):
            up = arr.copy()
            dn = arr.copy()
            up[i] = np.float32(arr[i] + h)
            dn[i] = np.float32(arr[i] - h)
            step = float(up[i]) - float(dn[i])         # the exact fp32 step taken
            if name == "H":
                fd[i] = (loss_at(up, x.W) - loss_at(dn, x.W)) / step
            else:
                fd[i] = (loss_at(x.H, up) - loss_at(x.H, dn)) / step
        assert _rel(fd, grad) <= 1e-6, name
    assert np.all(base["grad_H"][1] == 0.0)          # ignored row


# --------------------------------------------------------------------------
# closed forms: self-distillation and uniform student
# --------------------------------------------------------------------------
def _exact_grid_problem(T, d, V, seed):
    # values k/8 with small k: products and sums exact in fp32 and fp64
    rng = np.random.default_rng(seed)
    H = (rng.integers(-4, 5, size=(T, d)) / 8.0).astype(np.float32)
    W = (rng.integers(-4, 5, size=(V, d)) / 8.0).astype(np.float32)
    return H, W


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_self_distillation_closed_form(oracle, tau):
    T, d, V, K = 8, 6, 40, 7
    H, W = _exact_grid_problem(T, d, V, 21)
    z = H.astype(np.float64) @ W.astype(np.float64).T      # exact
    rng = np.random.default_rng(22)
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(T)]).astype(np.int32)
    lg = np.take_along_axis(z, idx.astype(np.int64), axis=1).astype(np.float32)
    r = oracle.full(H, W, idx, lg, None, tau=tau)
    logq = log_softmax(z / tau, axis=1)
    Q = np.exp(np.take_along_axis(logq, idx.astype(np.int64), axis=1)).sum(1)
    np.testing.assert_allclose(r["row_loss"], -np.log(Q), rtol=1e-12, atol=1e-15)
    # K = V: teacher == student, so loss and gradients vanish
    idxf = np.stack([rng.permutation(V) for _ in range(T)]).astype(np.int32)
    lgf = np.take_along_axis(z, idxf.astype(np.int64), axis=1).astype(np.float32)
    rf = oracle.full(H, W, idxf, lgf, None, tau=tau)
    assert abs(rf["loss"]) <= 1e-14
    assert np.max(np.abs(rf["grad_H"])) <= 1e-15
    assert np.max(np.abs(rf["grad_W"])) <= 1e-15


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_uniform_student_closed_form(oracle, tau):
    T, d, V, K = 10, 7, 53, 8
    x = _problem(T=T, d=d, V=V, K=K, tau=tau, seed=31, mask=("random", 0.2))
    W0 = np.zeros_like(x.W)
    r = oracle.full(x.H, W0, x.topk_idx, x.topk_logit, x.ignore, tau=tau)
    keep = x.ignore == 0
    N = keep.sum()
    p = softmax(x.topk_logit.astype(np.float64) / tau, axis=1)
    L = np.where(keep, math.log(V) - entropy(p, axis=1), 0.0)
    np.testing.assert_allclose(r["row_loss"], L, rtol=1e-12, atol=1e-15)
    assert abs(r["loss"] - L.sum() / N) <= 1e-12 * abs(r["loss"])
    assert np.all(r["grad_H"] == 0.0)
    s = 1.0 / (tau * N)
    Hk = x.H.astype(np.float64) * keep[:, None]
    gW = np.tile(s / V * Hk.sum(0), (V, 1))             # dense half: q = 1/V everywhere
    for t in range(T):                                  # sparse half: -P scattered at the ids
        if keep[t]:
            for k in range(K):
                gW[x.topk_idx[t, k]] -= s * p[t, k] * Hk[t]
    assert _rel(r["grad_W"], gW) <= 1e-12


# --------------------------------------------------------------------------
# temperature, mask, symmetries, upstream gradient
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tau", [2.0, 0.5])
def test_temperature_identity(oracle, tau):
    x = _problem(T=14, d=9, V=71, K=6, tau=tau, seed=41, mask=("random", 0.2))
    a = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=tau)
    W1 = (x.W / np.float32(tau)).astype(np.float32)          # exact: tau is a power of 2
    l1 = (x.topk_logit / np.float32(tau)).astype(np.float32)
    b = oracle.full(x.H, W1, x.topk_idx, l1, x.ignore, tau=1.0)
    assert abs(a["loss"] - b["loss"]) <= 1e-13 * abs(b["loss"])
    assert _rel(a["grad_H"], b["grad_H"]) <= 1e-12
    assert _rel(a["grad_W"], b["grad_W"] / tau) <= 1e-12


def test_mask_equals_deletion(oracle):
    T = 16
    x = _problem(T=T, d=8, V=45, K=5, tau=1.0, seed=51)
    ig = np.zeros(T, np.uint8)
    ig[[2, 9]] = 1
    m = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, ig, tau=1.0)
    keep = ig == 0
    dl = oracle.full(x.H[keep], x.W, x.topk_idx[keep], x.topk_logit[keep], None, tau=1.0)
    assert abs(m["loss"] - dl["loss"]) <= 1e-13 * abs(dl["loss"])
    assert _rel(m["grad_W"], dl["grad_W"]) <= 1e-13
    assert _rel(m["grad_H"][keep], dl["grad_H"]) <= 1e-13
    assert np.all(m["grad_H"][~keep] == 0.0)
    allm = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, np.ones(T, np.uint8), tau=1.0)
    assert allm["loss"] == 0.0
    assert np.all(allm["grad_H"] == 0.0) and np.all(allm["grad_W"] == 0.0)


def test_symmetries(oracle):
    T, V = 12, 41
    x = _problem(T=T, d=7, V=V, K=6, tau=1.0, seed=61, mask=("random", 0.2))
    base = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0)
    rng = np.random.default_rng(62)
    # permute the K entries of every row
    pk = np.stack([rng.permutation(x.K) for _ in range(T)])
    r = oracle.full(x.H, x.W, np.take_along_axis(x.topk_idx, pk, 1),
                    np.take_along_axis(x.topk_logit, pk, 1), x.ignore, tau=1.0)
    assert abs(r["loss"] - base["loss"]) <= 1e-13 * abs(base["loss"])
    assert _rel(r["grad_W"], base["grad_W"]) <= 1e-13
    # permute positions
    pt = rng.permutation(T)
    r = oracle.full(x.H[pt], x.W, x.topk_idx[pt], x.topk_logit[pt], x.ignore[pt], tau=1.0)
    assert abs(r["loss"] - base["loss"]) <= 1e-13 * abs(base["loss"])
    assert _rel(r["grad_H"], base["grad_H"][pt]) <= 1e-13
    assert _rel(r["grad_W"], base["grad_W"]) <= 1e-12
    # permute the vocabulary: row v of W moves to pv_inv[v]
    pv = rng.permutation(V)                      # new row i holds old row pv[i]
    inv = np.argsort(pv)
    r = oracle.full(x.H, x.W[pv], inv[x.topk_idx].astype(np.int32), x.topk_logit, x.ignore, tau=1.0)
    assert abs(r["loss"] - base["loss"]) <= 1e-13 * abs(base["loss"])
    assert _rel(r["grad_W"], base["grad_W"][pv]) <= 1e-12
    assert _rel(r["grad_H"], base["grad_H"]) <= 1e-12


def test_linear_in_upstream_gradient(oracle):
    x = _problem(T=10, d=6, V=29, K=5, tau=1.0, seed=71)
    a = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0, g=1.0)
    b = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0, g=-2.5)
    assert a["loss"] == b["loss"]
    assert _rel(b["grad_H"], -2.5 * a["grad_H"]) <= 1e-14
    assert _rel(b["grad_W"], -2.5 * a["grad_W"]) <= 1e-14


def test_gradient_identities(oracle):
    """sum_v grad_W[v] = 0 (each row of G sums to zero) and <grad_W, W> = <grad_H, H>."""
    x = _problem(T=20, d=9, V=57, K=6, tau=1.3, seed=81, mask=("random", 0.15))
    r = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.3)
    gw, gh = r["grad_W"], r["grad_H"]
    assert np.max(np.abs(gw.sum(0))) <= 1e-14 * max(1.0, np.abs(gw).max() * x.V)
    lhs = float((gw * x.W.astype(np.float64)).sum())
    rhs = float((gh * x.H.astype(np.float64)).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1e-30)


def test_two_oracles_agree():
    """The C loops and the matrix-product version agree on a problem with bf16
    operands, ignored rows, duplicate ids, -inf teacher logits, tau = 2 and a
    ragged last chunk, also when only some grad_W rows are requested."""
    from oracle import kd_oracle, kd_oracle_blas
    x = make_inputs(90, 40, 700, 24, tau=2.0, dtype="bf16", seed=91, mask=("random", 0.2), w_std=0.3)
    x.topk_idx[:, 7] = x.topk_idx[:, 3]
    x.topk_logit[5, 10:] = -np.inf
    a = kd_oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=2.0, g=0.5, chunk=32)
    b = kd_oracle_blas.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=2.0, g=0.5, chunk=32)
    assert abs(a["loss"] - b["loss"]) <= 1e-13 * abs(a["loss"])
    for k in ("lse", "row_loss", "grad_H", "grad_W"):
        assert _rel(b[k], a[k]) <= 1e-13, k
    sel = np.array([0, 5, int(x.topk_idx[0, 0]), 699])
    c = kd_oracle_blas.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=2.0, g=0.5, chunk=64, w_rows=sel)
    assert _rel(c["grad_W_rows"], a["grad_W"][sel]) <= 1e-13
    np.testing.assert_allclose(c["lse"], a["lse"], rtol=1e-14)
