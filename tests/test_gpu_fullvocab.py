"""Element-by-element parity at full vocabulary size, through the C ABI.

* A 201,088-token vocabulary with chunks of 8,192 positions: one chunk's G is
  8,192 x 201,216 bf16 = 3.3 GB, so the operand windows of both gradient
  contractions lie beyond 2^31 bytes (ids from 131,072 on sit at G offsets
  past 2 GiB).  Two wider vocabularies (300,000 with 4,096-row chunks,
  600,000 with 2,048) do the same on the engine's operand-ring schedule.  T = 8,300 leaves a ragged second chunk of 108 rows; d = 136
  puts a K tail inside the logits contraction's last step and d = 320 a
  partial hidden tile in both gradient contractions.  Fused and split entries
  are compared with the fp64 oracle in full (loss, lse, row losses, grad_H,
  grad_W), plus the below-contract diagnostics of the dense gradient terms.
* The Llama-3B-like workload (T = 8,192, d = 3,072, V = 128,256, K = 100,
  5% ignored, chunk 1,024) in full, both entries, in the configuration the
  benchmark times it in.

The oracle here is the matrix-product writing of the definition
(oracle/kd_oracle_blas.py), pinned against the C loops and the independent
pins in tests/test_oracle_pins.py.  The pages make the dense evaluation the
correctness baseline of the chunked variants (ai-thai.com/posts/846, section
"Fused Chunked KL Loss", item "Dense KL").
"""
import gc

import numpy as np
import pytest
import torch

from chunked_top_kl_head_amd import binding as B
from chunked_top_kl_head_amd import synth
from oracle import kd_oracle_blas

from .gpu_util import tol_for, upload
from .test_gpu_parity import check_against, diagnostics, run_all_paths

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


# name: (T, d, V, K, tau, mask, chunk, seed)
# 8,192-row chunks run every contraction on the engine's two-stage schedule;
# the wide-vocabulary cases put G beyond 2 GiB in chunks short enough for the
# operand ring (logits and grad_H up to 4,096 rows, grad_W up to 2,048).
WIDE_CASES = {
    "d136_ktail_mask": (8300, 136, 201088, 100, 1.0, ("random", 0.05), 8192, 121),
    "d320_mtail_tau2": (8300, 320, 201088, 100, 2.0, None, 8192, 122),
    "ring_lh_V300k": (4200, 64, 300000, 20, 1.0, ("random", 0.05), 4096, 123),
    "ring_all_V600k": (2100, 64, 600000, 20, 1.0, None, 2048, 124),
}


@pytest.mark.parametrize("name", list(WIDE_CASES))
def test_chunk_G_beyond_2GiB(name):
    T, d, V, K, tau, mask, chunk, seed = WIDE_CASES[name]
    say(f"case {name}: T={T} d={d} V={V} K={K} tau={tau} chunk={chunk} "
        f"(chunk G {chunk * ((V + 255) // 256 * 256) * 2 / 2**30:.2f} GiB)")
    x = synth.make_inputs(T, d, V, K, tau=tau, dtype="bf16", seed=seed, mask=mask)
    out = run_all_paths(upload(x), tau, chunk)
    say("  GPU done; oracle")
    ref = kd_oracle_blas.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=tau, chunk=1024)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for("bf16"), x, path)
    diagnostics(ref, out["fused"], x, tau)
    # ids whose G entries sit beyond 2 GiB of the blocked chunk buffer (element
    # (r, v) at ((v / 64) C + r) 64 + v % 64, two bytes each), on their own
    first_far = (1 << 30) // chunk
    assert first_far < V
    far = np.arange(first_far, V)
    for path in ("fused", "split"):
        e = np.max(np.abs(out[path]["grad_W"][far] - ref["grad_W"][far])) / np.max(np.abs(ref["grad_W"][far]))
        say(f"  {path}: grad_W rows of ids >= {first_far}, at their own scale: {e:.2e}")
        assert e <= 2e-2
    del out, ref
    gc.collect()
    torch.cuda.empty_cache()


def test_llama_workload_in_full():
    """Llama-3B-like workload: every output element of both entries against the oracle."""
    w = synth.WORKLOADS["llama3b"]
    say(f"workload llama3b: T={w.T} d={w.d} V={w.V} K={w.K} tau={w.tau} chunk={w.chunk} mask={w.mask}")
    x = synth.workload_inputs("llama3b")
    out = run_all_paths(upload(x), w.tau, w.chunk)
    torch.cuda.empty_cache()
    say("  GPU done; oracle")
    ref = kd_oracle_blas.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=w.tau, chunk=w.chunk)
    for path in ("fused", "split"):
        check_against(ref, out[path], tol_for("bf16"), x, path)
    diagnostics(ref, out["fused"], x, w.tau)
    del out, ref
    gc.collect()
