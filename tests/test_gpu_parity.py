"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Element-by-element comparisons run at sizes the oracle finishes in seconds but
that still span several output tiles, several chunks and ragged tails in every
dimension (rows, hidden size, vocabulary, chunk).  Edge cases: all positions
ignored, T = 0, one row, K = 1, K = V, duplicate ids, upstream gradient != 1.
"""
import numpy as np
import pytest
import torch

from chunked_top_kl_head_amd import binding as B
from chunked_top_kl_head_amd import synth

from .gpu_util import f64, loss_rel, rel_maxabs, tol_for, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_all_paths(dev, tau, chunk, grad_loss=None):
    """Fused entry, then forward + backward; returns host fp64 copies."""
    loss, gH, gW, lse, rl = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"],
                                               dev["ignore"], grad_loss=grad_loss, temperature=tau, chunk=chunk,
                                               want_lse=True, want_row_loss=True)
    floss, flse, frl = B.kd_topk_kl_forward(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], dev["ignore"],
                                            temperature=tau, chunk=chunk, want_row_loss=True)
    bgH, bgW = B.kd_topk_kl_backward(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], flse, dev["ignore"],
                                     grad_loss=grad_loss, temperature=tau, chunk=chunk)
    torch.cuda.synchronize()
    return dict(
        fused=dict(loss=float(loss.item()), grad_H=f64(gH), grad_W=f64(gW), lse=f64(lse), row_loss=f64(rl)),
        split=dict(loss=float(floss.item()), grad_H=f64(bgH), grad_W=f64(bgW), lse=f64(flse), row_loss=f64(frl)),
    )


def check_against(ref, out, tol, x, label):
    lr = loss_rel(out["loss"], ref["loss"])
    eH = rel_maxabs(out["grad_H"], ref["grad_H"])
    eW = rel_maxabs(out["grad_W"], ref["grad_W"])
    else_ = np.max(np.abs(out["lse"] - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))) if x.T else 0.0
    erow = np.max(np.abs(out["row_loss"] - ref["row_loss"]) / np.maximum(1.0, np.abs(ref["row_loss"]))) if x.T else 0.0
    say(f"  {label}: loss rel {lr:.2e}  grad_H {eH:.2e}  grad_W {eW:.2e}  lse {else_:.2e}  row {erow:.2e}")
    assert lr <= tol["loss"], (label, "loss", lr)
    assert eH <= tol["grad"], (label, "grad_H", eH)
    assert eW <= tol["grad"], (label, "grad_W", eW)
    assert else_ <= tol["lse"], (label, "lse", else_)
    assert erow <= tol["row"], (label, "row_loss", erow)


def diagnostics(ref, out, x, tau, g=1.0):
    """Checks below the contract's resolution: the dense (softmax) halves of the gradients.

    * grad_W rows of ids in no kept row's cache carry only the softmax term;
      compare them at their own scale.
    * grad_H + s * sum_k p_k W_idx_k is grad_H's softmax term; compare at its own scale.
    """
    keep = x.ignore == 0
    N = int(keep.sum())
    if N == 0:
        return
    hot = np.zeros(x.V, dtype=bool)
    hot[np.unique(x.topk_idx[keep])] = True
    cold = ~hot
    if cold.any():
        e = rel_maxabs(out["grad_W"][cold], ref["grad_W"][cold])
        say(f"  cold grad_W rows ({int(cold.sum())}): rel {e:.2e}")
        assert e <= 2e-2
    s = g / (tau * N)
    lg = x.topk_logit.astype(np.float64) / tau
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    sparse = np.zeros((x.T, x.d))
    qbound = np.zeros((x.T, x.d))
    Wd = x.W.astype(np.float64)
    Hd = x.H.astype(np.float64)
    for t in np.nonzero(keep)[0]:
        Wk = Wd[x.topk_idx[t]]
        sparse[t] = s * (p[t][:, None] * Wk).sum(0)
        q = np.exp(Wk @ Hd[t] / tau - ref["lse"][t])
        qbound[t] = (np.abs(s * (q - p[t]))[:, None] * np.abs(Wk)).sum(0)
    # With bf16 operands two roundings are discounted before the remaining
    # error is compared with the dense term's scale: grad_H's own output
    # rounding (<= 2^-8 |x|) and the bf16 rounding of G's cached-id entries
    # (<= 2^-8 |G_k|, summed against |W_k|); both are set by the sparse term,
    # which is much larger than the dense one.
    dense_ref = ref["grad_H"][keep] + sparse[keep]
    err = np.abs(out["grad_H"][keep] - ref["grad_H"][keep])
    if x.dtype == "bf16":
        err = np.maximum(0.0, err - 2.0 ** -8 * (np.abs(ref["grad_H"][keep]) + qbound[keep]))
    e = float(err.max() / np.abs(dense_ref).max())
    say(f"  dense part of grad_H (beyond output rounding): rel {e:.2e}")
    assert e <= 2e-2


SMALL_CASES = {
    # name: (T, d, V, K, tau, dtype, mask, chunk, seed)
    "bf16_ragged": (700, 320, 5000, 50, 1.0, "bf16", ("random", 0.1), 256, 101),
    "bf16_tau2_ktail": (333, 136, 3001, 100, 2.0, "bf16", ("random", 0.2), 128, 102),
    "f32_ragged": (300, 200, 1000, 16, 0.7, "f32", None, 96, 103),
}


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_small_parity(oracle, name):
    T, d, V, K, tau, dt, mask, chunk, seed = SMALL_CASES[name]
    say(f"case {name}: T={T} d={d} V={V} K={K} tau={tau} {dt} chunk={chunk}")
    x = synth.make_inputs(T, d, V, K, tau=tau, dtype=dt, seed=seed, mask=mask)
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=tau)
    out = run_all_paths(upload(x), tau, chunk)
    tol = tol_for(dt)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol, x, path)
    diagnostics(ref, out["fused"], x, tau)


# The bf16 engine runs a chunk's contractions on one of two schedules, chosen
# by the chunk's rows (the operand ring up to 4,096 rows for the logits and
# grad_H contractions and up to 2,048 for grad_W, the two-stage pipeline
# above).  These chunk sizes cross both switch points on small shapes with
# tails, so both schedules of every contraction meet the oracle:
#   4,608 rows: all three on the two-stage schedule, the ragged 92-row
#               remainder on the ring;
#   3,000 rows: logits and grad_H on the ring, grad_W on the two-stage one.
SWITCH_CASES = {
    # name: (T, d, V, K, tau, mask, chunk, seed)
    "two_stage_all_ktail": (4700, 136, 3001, 30, 1.5, ("random", 0.1), 4608, 105),
    "ring_lh_two_stage_w_mtail": (3100, 320, 3001, 30, 1.0, ("random", 0.05), 3000, 106),
}


@pytest.mark.parametrize("name", list(SWITCH_CASES))
def test_both_engine_schedules(name):
    from oracle import kd_oracle_blas

    T, d, V, K, tau, mask, chunk, seed = SWITCH_CASES[name]
    say(f"case {name}: T={T} d={d} V={V} K={K} tau={tau} bf16 chunk={chunk}")
    x = synth.make_inputs(T, d, V, K, tau=tau, dtype="bf16", seed=seed, mask=mask)
    out = run_all_paths(upload(x), tau, chunk)
    ref = kd_oracle_blas.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=tau)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for("bf16"), x, path)
    diagnostics(ref, out["fused"], x, tau)


def test_schedules_agree_bitwise_on_logits():
    """Both schedules accumulate the K steps of a tile in the same order, so a
    row's logits, hence its lse and row loss, are the same bits whichever
    schedule its chunk ran on: 4,608-row chunks (two-stage) against 1,024-row
    chunks (operand ring).  The two-stage run is also repeated bitwise."""
    T, d, V, K, tau, mask, _, seed = SWITCH_CASES["two_stage_all_ktail"]
    x = synth.make_inputs(T, d, V, K, tau=tau, dtype="bf16", seed=seed, mask=mask)
    dev = upload(x)

    def run(chunk):
        loss, gH, gW, lse, rl = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"],
                                                   dev["ignore"], temperature=tau, chunk=chunk, want_lse=True,
                                                   want_row_loss=True)
        torch.cuda.synchronize()
        return loss.clone(), gH.clone(), gW.clone(), lse.clone(), rl.clone()

    a, b, c = run(4608), run(4608), run(1024)
    for u, v in zip(a, b):
        assert torch.equal(u, v), "two-stage schedule not run-to-run deterministic"
    assert torch.equal(a[3].view(torch.int32), c[3].view(torch.int32)), "lse differs between schedules"
    assert torch.equal(a[4].view(torch.int32), c[4].view(torch.int32)), "row losses differ between schedules"
    say("  lse and row losses bitwise equal across schedules; two-stage repeat bitwise equal")


def _random_cases(n=24, seed=2026):
    """Seeded random shapes: hidden sizes 8..520 (K tails inside a step, partial
    hidden tiles), vocabularies that are not multiples of 4, chunks from one row
    to all rows, temperatures 0.5..3, random masks; bf16 and fp32."""
    rng = np.random.default_rng(seed)
    cases = {}
    for i in range(n):
        dt = "f32" if i % 4 == 3 else "bf16"
        T = int(rng.integers(1, 900))
        d = 8 * int(rng.integers(1, 66))
        V = int(rng.integers(40, 9000))
        K = int(rng.integers(1, min(200, V) + 1))
        chunk = 0 if i % 5 == 0 else int(rng.integers(1, T + 1))
        tau = round(float(rng.uniform(0.5, 3.0)), 3)
        mask = None if i % 3 == 0 else ("random", round(float(rng.uniform(0.0, 0.3)), 3))
        cases[f"r{i}_{dt}_T{T}_d{d}_V{V}_K{K}_c{chunk}"] = (T, d, V, K, tau, dt, mask, chunk, 200 + i)
    return cases


def _random_medium_cases(n=6, seed=2027):
    """Seeded random problems whose chunks (2,049 rows up to all of T) put grad_W,
    and above 4,096 rows the logits and grad_H contractions too, on the engine's
    two-stage schedule, with random hidden and vocabulary tails."""
    rng = np.random.default_rng(seed)
    cases = {}
    for i in range(n):
        T = int(rng.integers(4100, 5200))
        d = 8 * int(rng.integers(1, 48))
        V = int(rng.integers(300, 6000))
        K = int(rng.integers(1, min(120, V) + 1))
        chunk = int(rng.integers(2049, T + 1))
        tau = round(float(rng.uniform(0.5, 3.0)), 3)
        mask = ("random", round(float(rng.uniform(0.0, 0.2)), 3)) if i % 2 else None
        cases[f"m{i}_bf16_T{T}_d{d}_V{V}_K{K}_c{chunk}"] = (T, d, V, K, tau, "bf16", mask, chunk, 300 + i)
    return cases


RANDOM_CASES = {**_random_cases(), **_random_medium_cases()}


@pytest.mark.parametrize("name", list(RANDOM_CASES))
def test_random_shapes(name):
    from oracle import kd_oracle_blas

    T, d, V, K, tau, dt, mask, chunk, seed = RANDOM_CASES[name]
    say(f"case {name}: tau={tau} mask={mask}")
    x = synth.make_inputs(T, d, V, K, tau=tau, dtype=dt, seed=seed, mask=mask)
    out = run_all_paths(upload(x), tau, chunk)
    ref = kd_oracle_blas.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=tau)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for(dt), x, path)


def test_tiny_workload(oracle):
    """The smallest standard workload in full: fp32, T=256, d=256, V=4096, K=16, chunk 64."""
    w = synth.WORKLOADS["tiny"]
    say(f"workload tiny: T={w.T} d={w.d} V={w.V} K={w.K} chunk={w.chunk}")
    x = synth.workload_inputs("tiny")
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=w.tau)
    out = run_all_paths(upload(x), w.tau, w.chunk)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for(w.dtype), x, path)
    diagnostics(ref, out["fused"], x, w.tau)


def test_chunk_invariance_and_determinism(oracle):
    x = synth.make_inputs(640, 256, 4500, 40, tau=1.0, dtype="bf16", seed=104, mask=("random", 0.05))
    dev = upload(x)
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0)
    outs = {}
    for chunk in (128, 256, 640, 0):
        say(f"chunk {chunk}")
        loss, gH, gW, lse, _ = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"],
                                                  dev["ignore"], chunk=chunk, want_lse=True)
        torch.cuda.synchronize()
        outs[chunk] = (float(loss.item()), f64(gH), f64(gW), f64(lse))
        assert loss_rel(outs[chunk][0], ref["loss"]) <= 1e-3
        assert rel_maxabs(outs[chunk][1], ref["grad_H"]) <= 2e-2
        assert rel_maxabs(outs[chunk][2], ref["grad_W"]) <= 2e-2
    # lse does not depend on the chunking at all (row-local, same tiles)
    for c in (256, 640, 0):
        assert np.array_equal(outs[c][3], outs[128][3])
    # repeated call: bitwise identical
    loss2, gH2, gW2, _, _ = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"],
                                               dev["ignore"], chunk=256)
    torch.cuda.synchronize()
    assert float(loss2.item()) == outs[256][0]
    assert np.array_equal(f64(gH2), outs[256][1]) and np.array_equal(f64(gW2), outs[256][2])


def test_all_ignored_and_empty():
    x = synth.make_inputs(300, 64, 700, 8, dtype="bf16", seed=105, mask=("all",))
    dev = upload(x)
    say("all positions ignored")
    loss, gH, gW, lse, rl = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"],
                                               dev["ignore"], chunk=128, want_lse=True, want_row_loss=True)
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0
    assert torch.count_nonzero(gH).item() == 0 and torch.count_nonzero(gW).item() == 0
    assert torch.count_nonzero(rl).item() == 0
    assert torch.isfinite(lse).all()
    say("T = 0")
    e = synth.make_inputs(0, 64, 700, 8, dtype="bf16", seed=106)
    de = upload(e)
    gW0 = torch.full((700, 64), 7.0, device="cuda")
    loss, gH, gW, _, _ = B.kd_topk_kl_fused(de["H"], de["W"], de["topk_idx"], de["topk_logit"], None, grad_W=gW0)
    floss, flse, _ = B.kd_topk_kl_forward(de["H"], de["W"], de["topk_idx"], de["topk_logit"], None)
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0 and float(floss.item()) == 0.0
    assert torch.count_nonzero(gW).item() == 0 and gH.numel() == 0 and flse.numel() == 0


@pytest.mark.parametrize("shape", [(1, 64, 300, 7), (37, 64, 300, 1), (20, 72, 300, 300)],
                         ids=["one_row", "K1", "K_eq_V"])
def test_degenerate_shapes(oracle, shape):
    T, d, V, K = shape
    say(f"shape T={T} d={d} V={V} K={K}")
    x = synth.make_inputs(T, d, V, K, tau=1.0, dtype="bf16", seed=107, w_std=0.3)
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0)
    out = run_all_paths(upload(x), 1.0, 0)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for("bf16"), x, path)


def test_duplicate_ids_and_upstream_gradient(oracle):
    x = synth.make_inputs(200, 128, 2000, 12, tau=1.5, dtype="bf16", seed=108, w_std=0.2)
    x.topk_idx[:, 5] = x.topk_idx[:, 2]            # duplicates: P accumulates both entries
    x.topk_idx[7, :] = x.topk_idx[7, 0]            # one row of a single repeated id
    x.topk_logit[3, 4:] = -np.inf                  # zero-probability entries
    g = 2.5
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.5, g=g)
    gl = torch.tensor([g], dtype=torch.float32, device="cuda")
    say("duplicates + grad_loss 2.5")
    out = run_all_paths(upload(x), 1.5, 64, grad_loss=gl)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for("bf16"), x, path)


# (T, d, V, K, chunk, kept-row positions of the five planted rows).  "wide":
# a vocabulary of 70,000 ids cuts G into more spans than the rescale pass's
# grid has workgroups (1,024), so its workgroups stride over spans (bf16:
# ids from 65,536 on; fp32: each row's last span), and the last planted row
# sits in the second chunk.
RESCALE_CASES = {
    "narrow": (300, 320, 3000, 20, 128, (0, 40, -1, 100, 150)),
    "wide": (150, 64, 70000, 20, 128, (0, 40, -1, 60, 90)),
}


@pytest.mark.parametrize("case", list(RESCALE_CASES))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_far_above_their_cached_logits(oracle, dtype, case):
    """Rows whose largest student logit lies far above every cached id's.

    The fused entry stores each 128-id block's exponentials relative to the
    row's largest cached-id logit unless the block's own max exceeds it by more
    than 64 (base 2); such rows take the rescale path.  A vocabulary row planted
    as W_v = a H_t (v outside row t's cache) lifts z_tv to a |H_t|^2:
    z = 64 puts it ~92 (base 2) above the cached logits (rescaled rows), z = 38
    ~55 (stored values up to ~2^55 on the common path)."""
    T, d, V, K, chunk, at = RESCALE_CASES[case]
    x = synth.make_inputs(T, d, V, K, tau=1.0, dtype=dtype, seed=109, mask=("random", 0.1))
    kept = np.nonzero(x.ignore == 0)[0]
    plant = [(int(kept[at[0]]), 64.0), (int(kept[at[1]]), 64.0), (int(kept[at[2]]), 64.0),
             (int(kept[at[3]]), 38.0), (int(kept[at[4]]), 38.0)]
    used = set()
    W = x.W.copy()
    for t, z in plant:
        v = next(v for v in range(x.V - 1, -1, -1) if v not in set(x.topk_idx[t].tolist()) and v not in used)
        used.add(v)
        h = x.H[t].astype(np.float64)
        W[v] = (z / float(h @ h)) * x.H[t]
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(W.astype(np.float32))
        x.W_bits[:] = bits.reshape(x.W_bits.shape)
        x.W[:] = synth.bf16_bits_to_f32(bits).reshape(x.W.shape)
    else:
        x.W[:] = W
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0)
    gap = [(ref["lse"][t] - np.max(x.H[t].astype(np.float64) @ x.W[x.topk_idx[t]].astype(np.float64).T)) / np.log(2)
           for t, _ in plant]
    say("planted rows, lse above the best cached logit (base 2): " + " ".join(f"{g:.0f}" for g in gap))
    assert min(gap[:3]) > 70 and 40 < min(gap[3:]) < 64
    out = run_all_paths(upload(x), 1.0, chunk)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for(dtype), x, path)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ignored_row_with_very_negative_logits(oracle, dtype):
    """An ignored position whose every base-2 logit lies far below -126: its
    lse stays finite (it has no reference of its own) and the split
    backward's G row is exactly zero, so nothing non-finite reaches grad_W."""
    T, d, V, K = 300, 64, 3000, 20
    x = synth.make_inputs(T, d, V, K, tau=1.0, dtype=dtype, seed=110, mask=("random", 0.1))
    # every vocabulary row gets 2^-6 on hidden axis 0 (the size of its other
    # entries, so kept rows see an ordinary problem); one ignored row sits at
    # -2^15 on that axis, so all its logits are about -512 (exact in bf16)
    r = int(np.nonzero(x.ignore)[0][0])
    x.W[:, 0] = 2.0 ** -6
    x.H[r, 0] = -(2.0 ** 15)
    if dtype == "bf16":
        x.W_bits[:] = synth.f32_to_bf16_bits(x.W).reshape(x.W_bits.shape)
        x.H_bits[:] = synth.f32_to_bf16_bits(x.H).reshape(x.H_bits.shape)
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0)
    zmax = float(np.max(x.H[r].astype(np.float64) @ x.W.astype(np.float64).T))
    say(f"ignored row {r}: largest logit {zmax:.1f} (base 2: {zmax / np.log(2):.0f}), oracle lse {ref['lse'][r]:.2f}")
    assert zmax / np.log(2) < -600
    out = run_all_paths(upload(x), 1.0, 128)
    for path in ("fused", "split"):
        assert np.isfinite(out[path]["lse"]).all() and np.isfinite(out[path]["grad_W"]).all()
        assert np.all(out[path]["grad_H"][r] == 0.0)
        check_against(ref, out[path], tol_for(dtype), x, path)


def test_validate_counts_bad_cache():
    T, K, V = 50, 6, 100
    rng = np.random.default_rng(0)
    idx = rng.integers(0, V, size=(T, K)).astype(np.int32)
    lg = rng.standard_normal((T, K)).astype(np.float32)
    idx[3, 1] = V          # out of range
    idx[9, 0] = -4         # out of range
    lg[11, :] = -np.inf    # no finite teacher logit
    lg[12, 2] = np.nan     # NaN
    ig = np.zeros(T, np.uint8)
    ig[12] = 1             # ignored rows are not checked
    bad = B.kd_topk_kl_validate(torch.from_numpy(idx).cuda(), torch.from_numpy(lg).cuda(), V,
                                torch.from_numpy(ig).cuda())
    torch.cuda.synchronize()
    assert int(bad.item()) == 3
