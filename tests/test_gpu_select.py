"""GPU parity of the teacher top-K cache producer (kd_topk_select) against the
oracle (oracle/topk_select.py): ids and values bit for bit."""
import numpy as np
import pytest
import torch

from chunked_top_kl_head_amd import binding as B
from oracle.topk_select import topk_select

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_and_compare(x: np.ndarray, K: int, dtype, ld=None):
    """x: fp32 values (already bf16-representable when dtype is bf16)."""
    T, V = x.shape
    pitch = V if ld is None else ld
    host = np.zeros((T, pitch), dtype=np.float32)
    host[:, V:] = np.inf            # padding beyond V must never be selected
    host[:, :V] = x
    dev = torch.from_numpy(host).cuda().to(dtype)
    idx, val = B.kd_topk_select(dev, K, V=V)
    torch.cuda.synchronize()
    ref_idx, ref_val = topk_select(x, K)
    got_idx = idx.cpu().numpy()
    got_val = val.cpu().numpy()
    assert np.array_equal(got_idx, ref_idx)
    # values bit for bit (signed zeros included); a selected NaN is some NaN
    nan = np.isnan(ref_val)
    assert np.array_equal(np.isnan(got_val), nan)
    assert np.array_equal(got_val[~nan].view(np.uint32), ref_val[~nan].view(np.uint32))


def bf16_values(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("V,K", [(37, 1), (37, 37), (1000, 100), (5003, 100), (5003, 1024), (20000, 100)])
def test_random_rows(dtype, V, K):
    rng = np.random.default_rng(V * 7 + K)
    x = (rng.standard_normal((48, V)) * 3).astype(np.float32)
    if dtype == torch.bfloat16:
        x = bf16_values(x)
    say(f"V={V} K={K} {dtype}")
    run_and_compare(x, K, dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_special_rows(dtype):
    """Ties (candidate overflow: the exact path), sorted rows, constant rows,
    -inf, NaN and signed zeros, and a row pitch beyond V."""
    rng = np.random.default_rng(5)
    V = 4100
    rows = [
        rng.integers(0, 4, V).astype(np.float32),                   # 4 distinct values: heavy ties
        np.sort(rng.standard_normal(V)).astype(np.float32),        # ascending
        -np.sort(-rng.standard_normal(V)).astype(np.float32),      # descending
        np.zeros(V, np.float32),                                   # constant
        np.full(V, -np.inf, np.float32),
    ]
    r = rng.standard_normal(V).astype(np.float32)
    r[::5] = -np.inf
    r[2::9] = np.nan
    r[10], r[11], r[12] = 0.0, -0.0, 0.0
    rows.append(r)
    x = np.stack(rows)
    if dtype == torch.bfloat16:
        x = bf16_values(x)
    for K in (1, 100, 1024, V):
        if K <= 1024:
            run_and_compare(x, K, dtype)
    run_and_compare(x, 100, dtype, ld=V + 60)


def test_full_size_teacher_cache():
    """The 32,768 x 201,088 bf16 teacher logits of the GPT-OSS-like workload,
    K = 100: sampled rows against the oracle, every row checked for order."""
    T, V, K = 32768, 201088, 100
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    logits = (torch.randn(T, V, device="cuda", generator=g) * 3).to(torch.bfloat16)
    idx, val = B.kd_topk_select(logits, K)
    torch.cuda.synchronize()
    # every row: descending, values are the logits at the ids
    assert bool((val[:, 1:] <= val[:, :-1]).all())
    assert torch.equal(torch.gather(logits, 1, idx.long()).float(), val)
    rows = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(1).choice(T, 29, replace=False)]))
    sub = logits[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref_idx, ref_val = topk_select(sub, K)
    assert np.array_equal(idx[torch.from_numpy(rows).cuda()].cpu().numpy(), ref_idx)
    assert np.array_equal(val[torch.from_numpy(rows).cuda()].cpu().numpy(), ref_val)
    say(f"  {rows.size} sampled rows exact; all {T} rows ordered")


# ---------------------------------------------------------------------------
# kd_teacher_topk: the cache straight from the teacher's hidden states.  The
# logits are fp32 sums of d products, so near-ties at the K-th value may be
# ordered either way: what is unique is checked exactly (every id far enough
# above the K-th logit is kept, nothing far below it is), the rest for
# validity (distinct ids in range, values = the logits at the ids within the
# fp32 summation bound, descending).
# ---------------------------------------------------------------------------
def check_teacher(H64, W64, idx, val, K):
    d = H64.shape[1]
    z = H64 @ W64.T
    bound = (np.abs(H64) @ np.abs(W64).T) * (d * 2.0 ** -24) + 1e-30
    T, V = z.shape
    assert idx.shape == (T, K) and val.shape == (T, K)
    for t in range(T):
        ids = idx[t].astype(np.int64)
        assert np.all((ids >= 0) & (ids < V)) and np.unique(ids).size == K
        assert np.all(np.abs(val[t].astype(np.float64) - z[t, ids]) <= bound[t, ids])
        assert np.all(val[t, :-1] >= val[t, 1:])
        zK = np.partition(z[t], V - K)[V - K]          # K-th largest logit
        margin = 2.0 * bound[t].max()
        assert np.all(z[t, ids] >= zK - margin)
        must = np.nonzero(z[t] > zK + margin)[0]
        assert np.isin(must, ids).all()


# bf16 operands go through the select that reads only the 128-id blocks whose
# record reaches the bound (with K above the number of blocks, or too many
# candidates, it takes every block and may finish with the exact full-row
# select); fp32 operands through the full-row select.
@pytest.mark.parametrize("dtype,T,d,V,K,chunk", [
    ("bf16", 300, 256, 5000, 20, 128),     # three chunks, the last ragged; vocabulary tail in the last tile
    ("bf16", 200, 136, 20000, 100, 64),    # K close to the number of blocks (157)
    ("bf16", 70, 136, 3001, 100, 0),       # V not a multiple of 4 (padded rows of the chunk buffer); K > blocks
    ("bf16", 33, 64, 37, 37, 16),          # K = V
    ("bf16", 4700, 136, 3001, 20, 4608),   # a chunk above 4,096 rows: the two-stage schedule, then the ring
    ("f32", 130, 64, 3000, 10, 64),
    ("f32", 100, 64, 1000, 10, 64),
])
def test_teacher_topk(dtype, T, d, V, K, chunk):
    from chunked_top_kl_head_amd import synth
    x = synth.make_inputs(T, d, V, K, tau=1.0, dtype=dtype, seed=31, mask=None)
    if dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).cuda().view(torch.bfloat16)
        W = torch.from_numpy(x.W_bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        H = torch.from_numpy(x.H).cuda()
        W = torch.from_numpy(x.W).cuda()
    idx, val = B.kd_teacher_topk(H, W, K, chunk=chunk)
    torch.cuda.synchronize()
    check_teacher(x.H.astype(np.float64), x.W.astype(np.float64), idx.cpu().numpy(), val.cpu().numpy(), K)
    say(f"  teacher top-{K}: {dtype} T={T} d={d} V={V} chunk={chunk} ok")


def test_teacher_topk_full_size():
    """GPT-OSS-like teacher shapes (T = 32,768, d = 2,880, V = 201,088, K = 100,
    bf16): every row ordered with distinct ids; 24 sampled rows against the
    fp64 oracle."""
    from chunked_top_kl_head_amd import synth
    x = synth.workload_inputs("gptoss20b")
    H = torch.from_numpy(x.H_bits.view(np.int16)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(x.W_bits.view(np.int16)).cuda().view(torch.bfloat16)
    K = 100
    idx, val = B.kd_teacher_topk(H, W, K)
    torch.cuda.synchronize()
    assert bool((val[:, 1:] <= val[:, :-1]).all())
    s, _ = torch.sort(idx, dim=1)
    assert bool((s[:, 1:] != s[:, :-1]).all()) and int(idx.min()) >= 0 and int(idx.max()) < x.V
    rows = np.unique(np.concatenate([[0, x.T - 1], np.random.default_rng(3).choice(x.T, 22, replace=False)]))
    r = torch.from_numpy(rows).cuda()
    check_teacher(x.H[rows].astype(np.float64), x.W.astype(np.float64), idx[r].cpu().numpy(), val[r].cpu().numpy(), K)
    say(f"  {rows.size} sampled rows valid; all {x.T} rows ordered")


def test_teacher_topk_heavy_ties():
    """Every vocabulary row is one of three rows, so each position's logits take
    three values, each on a third of the ids: every 128-id block reaches the
    K-th largest block maximum and the candidates (3,000 equal logits) overflow
    the buffer, which sends the rows to the exact full-row select.  The answer
    is unique: the K smallest ids of the class with the largest logit."""
    T, d, V, K = 40, 64, 9000, 50
    rng = np.random.default_rng(11)
    base = (rng.standard_normal((3, d)) * 0.05).astype(np.float32)
    Hf = rng.standard_normal((T, d)).astype(np.float32)
    Wf = base[np.arange(V) % 3]
    from chunked_top_kl_head_amd import synth
    H = torch.from_numpy(synth.f32_to_bf16_bits(Hf).view(np.int16).reshape(T, d)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(synth.f32_to_bf16_bits(Wf).view(np.int16).reshape(V, d)).cuda().view(torch.bfloat16)
    idx, val = B.kd_teacher_topk(H, W, K, chunk=16)
    torch.cuda.synchronize()
    H64 = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(Hf)).reshape(T, d).astype(np.float64)
    b64 = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(base)).reshape(3, d).astype(np.float64)
    z = H64 @ b64.T                                   # [T, 3]
    srt = np.sort(z, axis=1)
    clear = (srt[:, 2] - srt[:, 1]) > 1e-3 * np.abs(srt[:, 2]).max()
    idx_h, val_h = idx.cpu().numpy(), val.cpu().numpy()
    for t in np.nonzero(clear)[0]:
        c = int(np.argmax(z[t]))
        expect = np.arange(c, V, 3)[:K]
        assert np.array_equal(idx_h[t], expect), t
        assert np.all(val_h[t] == val_h[t, 0])
    say(f"  heavy ties: {int(clear.sum())} of {T} rows checked exactly")
