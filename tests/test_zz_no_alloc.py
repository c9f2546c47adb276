"""The no-allocation fused entry (kd_topk_kl_fused_noalloc) against the fused
entry with a workspace, through the C ABI.

Two calls in a row on the library's static scratch, the second with a
smaller problem (the scratch still holds the first call's contents): with
the same chunk the two entries run the same kernels on the same data, so the
outputs must be bitwise identical.  With chunk = 0 the entry picks a chunk
that fits its 256 MiB scratch (a few hundred rows at a 201,088-token
vocabulary), so its results differ from the default-chunk fused entry only
by the grouping of grad_W's accumulation: they are compared at the parity
bars (loss relative error <= 1e-3, gradients <= 2e-2 max|ref|, lse bitwise:
it does not depend on the chunking).  An explicit chunk too large for the
scratch is rejected before anything runs.
"""
import numpy as np
import pytest
import torch

from chunked_top_kl_head_amd import binding as B
from chunked_top_kl_head_amd import synth

from .gpu_util import f64, loss_rel, rel_maxabs, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def outputs(x, dev):
    T, d, V = x.T, x.d, x.V
    return dict(loss=torch.empty(1, dtype=torch.float32, device=dev), grad_H=torch.empty((T, d), dtype=torch.bfloat16,
                device=dev), grad_W=torch.empty((V, d), dtype=torch.float32, device=dev),
                lse=torch.empty(T, dtype=torch.float32, device=dev), row_loss=torch.empty(T, dtype=torch.float32,
                device=dev))


def run_noalloc(x, d_in, out, chunk, g=None):
    B.kd_topk_kl_fused_noalloc(d_in["H"], d_in["W"], d_in["topk_idx"], d_in["topk_logit"], d_in["ignore"],
                               grad_loss=g, temperature=x.tau, chunk=chunk, **out)


def run_fused(x, d_in, chunk, g=None):
    loss, gH, gW, lse, rl = B.kd_topk_kl_fused(d_in["H"], d_in["W"], d_in["topk_idx"], d_in["topk_logit"],
                                               d_in["ignore"], grad_loss=g, temperature=x.tau, chunk=chunk,
                                               want_lse=True, want_row_loss=True)
    return dict(loss=loss, grad_H=gH, grad_W=gW, lse=lse, row_loss=rl)


def test_noalloc_matches_fused_entry_two_calls():
    dev = torch.device("cuda")
    g = torch.tensor([1.5], device=dev)
    # (T, d, V, K, tau, chunk, seed): the second call is smaller in every dimension
    for i, (T, d, V, K, tau, chunk, seed) in enumerate([(700, 320, 5000, 50, 1.0, 256, 301),
                                                        (130, 136, 3001, 20, 2.0, 64, 302)]):
        say(f"call {i + 1}: T={T} d={d} V={V} K={K} tau={tau} chunk={chunk}")
        x = synth.make_inputs(T, d, V, K, tau=tau, dtype="bf16", seed=seed, mask=("random", 0.1))
        d_in = upload(x)
        out = outputs(x, dev)
        before = torch.cuda.memory_allocated()
        run_noalloc(x, d_in, out, chunk, g)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        ref = run_fused(x, d_in, chunk, g)
        torch.cuda.synchronize()
        for k in ("loss", "grad_H", "grad_W", "lse", "row_loss"):
            assert torch.equal(out[k], ref[k]), (i, k)
        say(f"  bitwise equal to the fused entry (loss {float(out['loss'].item()):.6f})")


def test_noalloc_default_chunk_fits_the_scratch_at_full_vocabulary():
    dev = torch.device("cuda")
    T, d, V, K = 1500, 256, 201088, 100
    x = synth.make_inputs(T, d, V, K, tau=1.0, dtype="bf16", seed=303, mask=("random", 0.05))
    d_in = upload(x)
    prob = B.problem(T, d, V, K, 1.0, torch.bfloat16, 0)
    assert B.workspace_size(prob, B.KD_OP_FUSED) > 256 << 20      # the default chunk would not fit
    out = outputs(x, dev)
    run_noalloc(x, d_in, out, 0)
    ref = run_fused(x, d_in, 0)
    torch.cuda.synchronize()
    lr = loss_rel(float(out["loss"].item()), float(ref["loss"].item()))
    eH = rel_maxabs(f64(out["grad_H"]), f64(ref["grad_H"]))
    eW = rel_maxabs(f64(out["grad_W"]), f64(ref["grad_W"]))
    say(f"  chunk 0 vs fused default chunk: loss rel {lr:.2e}  grad_H {eH:.2e}  grad_W {eW:.2e}")
    assert torch.equal(out["lse"], ref["lse"])
    assert lr <= 1e-3 and eH <= 2e-2 and eW <= 2e-2
    # an explicit chunk whose workspace exceeds the scratch: rejected, outputs untouched
    out2 = outputs(x, dev)
    for t in out2.values():
        t.fill_(7.0)
    with pytest.raises(B.KdError) as e:
        run_noalloc(x, d_in, out2, 8192)
    assert e.value.status == B.KD_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in out2.values())
