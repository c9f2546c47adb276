"""Full-size checks at the standard workloads, in the configuration bench.py times.

The fp64 oracle cannot evaluate every gradient of a 32K x 201K problem in test
time, so at these sizes:
* sampled rows (first/last rows, chunk boundaries, ignored rows, seeded random
  rows) are compared one by one with the oracle's row-local quantities: lse,
  row loss and grad_H;
* the loss is checked to be the mean of the row losses over kept positions;
* grad_W is checked through identities that hold at any size:
    sum_v grad_W[v, :] = sum_t H_t (sum_v G_tv) = 0, and
    <grad_W, W> = sum_tv G_tv z_tv = <grad_H, H>;
* at the headline size (GPT-OSS-20B-like, T = 32,768, V = 201,088, chunks of
  8,192) the loss, every position's lse and row loss, and sampled grad_W rows
  (spread over the vocabulary, half of them ids whose entries in the chunk's
  G lie beyond 2 GiB) are compared element by element with the oracle.
The Llama-3B-like workload is compared in full in test_gpu_fullvocab.py.
"""
import gc

import numpy as np
import pytest
import torch

from chunked_top_kl_head_amd import binding as B
from chunked_top_kl_head_amd import synth
from oracle import kd_oracle_blas

from .gpu_util import upload

pytestmark = pytest.mark.gpu

N_RANDOM_ROWS = 16


def say(*a):
    print(*a, flush=True)


def sample_rows(x, chunk, seed):
    """First and last rows, the boundaries of the first two and the last chunk,
    some ignored rows and seeded random rows (about 30 rows in all)."""
    T = x.T
    rows = {0, 1, chunk - 1, chunk, 2 * chunk - 1, 2 * chunk, T - chunk - 1, T - chunk, T - 2, T - 1}
    rows = [r for r in rows if 0 <= r < T]
    rng = np.random.default_rng(seed)
    masked = np.nonzero(x.ignore)[0]
    if masked.size:
        rows += list(rng.choice(masked, size=min(3, masked.size), replace=False))
    rows += list(rng.choice(T, size=N_RANDOM_ROWS, replace=False))
    return np.array(sorted(set(int(r) for r in rows)), dtype=np.int64)


@pytest.mark.parametrize("name", ["gptoss20b", "batched4x32k", "extreme256k"])
def test_full_size_workload(oracle, name):
    w = synth.WORKLOADS[name]
    say(f"workload {name}: T={w.T} d={w.d} V={w.V} K={w.K} tau={w.tau} chunk={w.chunk} mask={w.mask}")
    x = synth.workload_inputs(name)
    dev = upload(x)
    loss, gH, gW, lse, rl = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"],
                                               dev["ignore"], temperature=w.tau, chunk=w.chunk,
                                               want_lse=True, want_row_loss=True)
    torch.cuda.synchronize()
    say("  fused call done")
    loss = float(loss.item())
    lse_h = lse.double().cpu().numpy()
    rl_h = rl.double().cpu().numpy()
    keep = x.ignore == 0
    N = int(keep.sum())

    # loss = mean of row losses over kept positions; ignored rows contribute 0
    assert np.all(rl_h[~keep] == 0.0)
    mean = rl_h[keep].sum() / N
    assert abs(loss - mean) <= 1e-5 * abs(mean), (loss, mean)

    # sampled rows against the oracle
    rows = sample_rows(x, w.chunk, seed=w.seed_index)
    ref = oracle.rows(rows, x.H[rows], x.W, x.topk_idx[rows], x.topk_logit[rows], x.ignore, x.T, tau=w.tau)
    e_lse = np.max(np.abs(lse_h[rows] - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"])))
    e_row = np.max(np.abs(rl_h[rows] - ref["row_loss"]) / np.maximum(1.0, np.abs(ref["row_loss"])))
    gH_rows = gH[torch.from_numpy(rows).to(gH.device)].double().cpu().numpy()
    e_gh = np.max(np.abs(gH_rows - ref["grad_H"])) / max(np.max(np.abs(ref["grad_H"])), 1e-30)
    say(f"  {rows.size} sampled rows: lse {e_lse:.2e}  row loss {e_row:.2e}  grad_H {e_gh:.2e}  loss {loss:.6f}")
    assert e_lse <= 1e-4
    assert e_row <= 1e-3
    assert e_gh <= 2e-2
    # the sampled kept rows' loss terms are also the oracle's
    kept_rows = rows[keep[rows]]
    assert np.all(np.abs(rl_h[kept_rows] - ref["row_loss"][keep[rows]]) <= 1e-3 * np.maximum(1.0, ref["row_loss"][keep[rows]]))

    # grad_W identities (fp64 on the host)
    gW_h = gW.double().cpu().numpy()
    col = gW_h.sum(axis=0)
    col_scale = np.abs(gW_h).sum(axis=0).max()
    r_col = float(np.abs(col).max() / col_scale)
    Hd = x.H.astype(np.float64)
    lhs = float(np.einsum("vd,vd->", gW_h, x.W.astype(np.float64)))
    rhs = float(np.einsum("td,td->", gH.double().cpu().numpy(), Hd))
    r_ip = abs(lhs - rhs) / max(abs(rhs), 1e-30)
    say(f"  grad_W column sums / scale {r_col:.2e};  <grad_W,W> {lhs:.6e} vs <grad_H,H> {rhs:.6e} (rel {r_ip:.2e})")
    assert r_col <= 5e-2
    assert r_ip <= 1e-2
    assert np.isfinite(gW_h).all()
    del gW_h, gH_rows, dev, gH, gW
    gc.collect()
    torch.cuda.empty_cache()


def test_headline_loss_lse_and_sampled_grad_W_rows():
    """GPT-OSS-20B-like workload as benched: loss, lse and row losses of all
    32,768 positions, and 48 grad_W rows, element by element against the oracle."""
    w = synth.WORKLOADS["gptoss20b"]
    say(f"workload gptoss20b: T={w.T} d={w.d} V={w.V} K={w.K} chunk={w.chunk}")
    x = synth.workload_inputs("gptoss20b")
    dev = upload(x)
    loss, gH, gW, lse, rl = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"],
                                               dev["ignore"], temperature=w.tau, chunk=w.chunk,
                                               want_lse=True, want_row_loss=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2026)
    fixed = [0, 1, 2, 99, 1000, 65535, 65536, 131071, 131072, 131073, 150000, w.V - 2, w.V - 1]
    sel = np.unique(np.concatenate([fixed, rng.integers(0, 131072, 12), rng.integers(131072, w.V, 24)]))
    gw_sel = gW[torch.from_numpy(sel).to(gW.device)].double().cpu().numpy()
    loss = float(loss.item())
    lse_h = lse.double().cpu().numpy()
    rl_h = rl.double().cpu().numpy()
    del dev, gH, gW, lse, rl
    gc.collect()
    torch.cuda.empty_cache()
    say(f"  GPU done; oracle over all positions ({sel.size} grad_W rows)")
    ref = kd_oracle_blas.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=w.tau, chunk=1024, w_rows=sel)
    e_loss = abs(loss - ref["loss"]) / abs(ref["loss"])
    e_lse = np.max(np.abs(lse_h - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"])))
    e_row = np.max(np.abs(rl_h - ref["row_loss"]) / np.maximum(1.0, np.abs(ref["row_loss"])))
    e_gw = np.max(np.abs(gw_sel - ref["grad_W_rows"])) / np.max(np.abs(ref["grad_W_rows"]))
    hot = np.isin(sel, x.topk_idx[x.ignore == 0])
    cold = ~hot
    e_cold = (np.max(np.abs(gw_sel[cold] - ref["grad_W_rows"][cold])) / np.max(np.abs(ref["grad_W_rows"][cold]))
              if cold.any() else 0.0)
    far = sel >= 131072
    e_far = np.max(np.abs(gw_sel[far] - ref["grad_W_rows"][far])) / np.max(np.abs(ref["grad_W_rows"][far]))
    say(f"  loss rel {e_loss:.2e}  lse {e_lse:.2e}  row loss {e_row:.2e}  grad_W rows {e_gw:.2e}  "
        f"(cold rows {int(cold.sum())}: {e_cold:.2e}; ids >= 131072: {e_far:.2e})")
    assert e_loss <= 1e-3
    assert e_lse <= 1e-4
    assert e_row <= 1e-3
    assert e_gw <= 2e-2
    assert e_cold <= 2e-2
    assert e_far <= 2e-2


def test_peak_hbm_linear_in_positions():
    """Peak device memory of a fused call (inputs + outputs + workspace) is affine in T."""
    d, V, K, chunk = 2880, 201088, 100, 4096
    dev = torch.device("cuda")
    W = (torch.randn(V, d, device=dev) * 0.02).to(torch.bfloat16)
    peaks = []
    Ts = [32768, 65536, 131072, 262144]
    gW = torch.empty(V, d, dtype=torch.float32, device=dev)
    for T in Ts:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        H = torch.randn(T, d, device=dev).to(torch.bfloat16)
        idx = torch.randint(0, V, (T, K), device=dev, dtype=torch.int32)
        lg = torch.randn(T, K, device=dev)
        loss, gH, _, _, _ = B.kd_topk_kl_fused(H, W, idx, lg, None, chunk=chunk, grad_W=gW)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        peaks.append(peak)
        say(f"  T={T}: peak above resident W/grad_W {peak / 2**30:.3f} GiB")
        del H, idx, lg, loss, gH
    Ts_a = np.array(Ts, dtype=np.float64)
    P = np.array(peaks, dtype=np.float64)
    beta, alpha = np.polyfit(Ts_a, P, 1)
    resid = np.max(np.abs(P - (alpha + beta * Ts_a)) / P)
    say(f"  slope {beta:.1f} B/token, intercept {alpha / 2**30:.3f} GiB, max residual {resid:.2e}")
    assert resid <= 1e-2
    # per-token bytes: H and grad_H (bf16) plus the cache (int32 ids, fp32 logits)
    expect = 2 * d * 2 + K * 8
    assert abs(beta - expect) <= 0.05 * expect
    # the workspace does not grow with T: the intercept is about one chunk's G
    assert alpha <= 3.0 * chunk * ((V + 255) // 256 * 256) * 2
