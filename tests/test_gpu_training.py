"""GPU checks of the training-step integration: the autograd function (both
modes, a retained graph differentiated twice, inputs that need no gradient),
grad_W accumulation into a caller's buffer, a bf16 teacher-logit cache and
gradient scaling in place and into fresh (bf16) outputs -- each against the
fp64 oracle.
"""
import numpy as np
import pytest
import torch

from chunked_top_kl_head_amd import binding as B
from chunked_top_kl_head_amd import synth
from chunked_top_kl_head_amd.autograd import topk_kl_loss

from .gpu_util import BF16_TOL, f64, loss_rel, rel_maxabs, upload

pytestmark = pytest.mark.gpu

# several chunks, ragged rows / hidden size / vocabulary, 10% ignored
SHAPE = dict(T=600, d=200, V=3000, K=40)
CHUNK = 256


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def problem(oracle):
    x = synth.make_inputs(SHAPE["T"], SHAPE["d"], SHAPE["V"], SHAPE["K"], tau=1.5, dtype="bf16", seed=201,
                          mask=("random", 0.1))
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.5)
    return x, ref


def check(label, loss, gH, gW, ref, g=1.0):
    lr = loss_rel(loss, ref["loss"])
    eH = rel_maxabs(gH, g * ref["grad_H"])
    eW = rel_maxabs(gW, g * ref["grad_W"])
    say(f"  {label}: loss rel {lr:.2e}  grad_H {eH:.2e}  grad_W {eW:.2e}")
    assert lr <= BF16_TOL["loss"] and eH <= BF16_TOL["grad"] and eW <= BF16_TOL["grad"]


@pytest.mark.parametrize("mode", ["fused", "recompute"])
def test_autograd_matches_oracle(problem, mode):
    x, ref = problem
    dev = upload(x)
    H = dev["H"].clone().requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    ign = torch.from_numpy(x.ignore).cuda()
    loss = topk_kl_loss(H, W, dev["topk_idx"], dev["topk_logit"], ign, temperature=1.5, chunk=CHUNK, mode=mode)
    (3.0 * loss).backward()      # upstream gradient 3
    torch.cuda.synchronize()
    assert H.grad.dtype == H.dtype and W.grad.dtype == W.dtype
    check(f"autograd {mode}, g = 3", float(loss.item()), f64(H.grad), f64(W.grad), ref, g=3.0)


def test_autograd_leading_dims_and_int64_ids(problem):
    """[B, S, d] hidden states and the int64 ids torch.topk returns."""
    x, ref = problem
    dev = upload(x)
    T, d = x.T, x.d
    H = dev["H"].clone().reshape(2, T // 2, d).requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    idx = dev["topk_idx"].to(torch.int64).reshape(2, T // 2, -1)
    lg = dev["topk_logit"].reshape(2, T // 2, -1)
    ign = torch.from_numpy(x.ignore).cuda().reshape(2, T // 2)
    loss = topk_kl_loss(H, W, idx, lg, ign, temperature=1.5, chunk=CHUNK)
    loss.backward()
    torch.cuda.synchronize()
    assert H.grad.shape == H.shape
    check("autograd [B, S, d]", float(loss.item()), f64(H.grad).reshape(T, d), f64(W.grad), ref)


@pytest.mark.parametrize("entry", ["fused", "backward"])
def test_accumulate_grad_W(problem, entry):
    x, ref = problem
    dev = upload(x)
    ign = torch.from_numpy(x.ignore).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    R = torch.randn(x.V, x.d, device="cuda", generator=gen) * float(np.abs(ref["grad_W"]).max())
    gW = R.clone()
    if entry == "fused":
        loss, gH, gW, _, _ = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], ign,
                                                temperature=1.5, chunk=CHUNK, grad_W=gW, accumulate=True)
        lval = float(loss.item())
    else:
        loss, lse, _ = B.kd_topk_kl_forward(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], ign,
                                            temperature=1.5, chunk=CHUNK)
        gH, gW = B.kd_topk_kl_backward(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], lse, ign,
                                       temperature=1.5, chunk=CHUNK, grad_W=gW, accumulate=True)
        lval = float(loss.item())
    torch.cuda.synchronize()
    check(f"accumulate ({entry})", lval, f64(gH), f64(gW) - f64(R), ref)


def test_accumulate_with_no_positions_leaves_grad_W():
    W = torch.randn(300, 64, device="cuda").to(torch.bfloat16)
    H = torch.empty(0, 64, device="cuda", dtype=torch.bfloat16)
    idx = torch.empty(0, 4, device="cuda", dtype=torch.int32)
    lg = torch.empty(0, 4, device="cuda", dtype=torch.float32)
    R = torch.randn(300, 64, device="cuda")
    gW = R.clone()
    B.kd_topk_kl_fused(H, W, idx, lg, None, grad_W=gW, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(gW, R)


def test_bf16_teacher_cache(oracle):
    """Teacher logits stored as bf16: the library widens them exactly, so the
    oracle on the same rounded values is the reference."""
    x = synth.make_inputs(500, 136, 2500, 30, tau=1.0, dtype="bf16", seed=202, mask=("random", 0.05))
    lg16 = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x.topk_logit)).reshape(x.topk_logit.shape)
    x.topk_logit[:] = lg16
    x.topk_logit[3, 5] = -np.inf          # a -inf entry survives the narrowing
    ref = oracle.full(x.H, x.W, x.topk_idx, x.topk_logit, x.ignore, tau=1.0)
    dev = upload(x)
    lg_bf16 = dev["topk_logit"].to(torch.bfloat16)
    assert torch.equal(lg_bf16.float(), dev["topk_logit"])      # exact
    ign = torch.from_numpy(x.ignore).cuda()
    loss, gH, gW, lse, _ = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], lg_bf16, ign, chunk=128,
                                              want_lse=True)
    torch.cuda.synchronize()
    check("bf16 cache (fused)", float(loss.item()), f64(gH), f64(gW), ref)
    l2, lse2, _ = B.kd_topk_kl_forward(dev["H"], dev["W"], dev["topk_idx"], lg_bf16, ign, chunk=128)
    torch.cuda.synchronize()
    assert float(l2.item()) == float(loss.item()) and torch.equal(lse, lse2)
    # validate reads the bf16 cache too: one kept row made all -inf
    bad_row = int(np.nonzero(x.ignore == 0)[0][0])
    lg_bad = lg_bf16.clone()
    lg_bad[bad_row] = float("-inf")
    assert int(B.kd_topk_kl_validate(dev["topk_idx"], lg_bad, x.V, ign).item()) == 1
    assert int(B.kd_topk_kl_validate(dev["topk_idx"], lg_bf16, x.V, ign).item()) == 0


def test_scale_grads_matches_upstream_gradient(problem):
    x, ref = problem
    dev = upload(x)
    ign = torch.from_numpy(x.ignore).cuda()
    g = torch.tensor([2.5], device="cuda")
    _, gH1, gW1, _, _ = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], ign,
                                           temperature=1.5, chunk=CHUNK)
    B.kd_topk_kl_scale_grads(g, gH1, gW1)           # in place
    loss, gH2, gW2, _, _ = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], ign,
                                              grad_loss=g, temperature=1.5, chunk=CHUNK)
    torch.cuda.synchronize()
    check("scaled after the fact, g = 2.5", float(loss.item()), f64(gH1), f64(gW1), ref, g=2.5)
    # the two differ only by where g meets the bf16 roundings: of G (grad_W)
    # and of G and the bf16 grad_H, rounded once more after scaling (<= 2^-8
    # of the largest element each)
    assert rel_maxabs(f64(gW1), f64(gW2)) <= 4e-3
    assert rel_maxabs(f64(gH1), f64(gH2)) <= 3 * 2.0 ** -8


@pytest.mark.parametrize("mode", ["fused", "recompute"])
def test_autograd_retained_graph_two_backwards(problem, mode):
    """(a * loss).backward(retain_graph=True) then (b * loss).backward(): each
    call's gradients are the oracle's times its own upstream gradient."""
    x, ref = problem
    dev = upload(x)
    H = dev["H"].clone().requires_grad_(True)
    W = dev["W"].clone().requires_grad_(True)
    ign = torch.from_numpy(x.ignore).cuda()
    loss = topk_kl_loss(H, W, dev["topk_idx"], dev["topk_logit"], ign, temperature=1.5, chunk=CHUNK, mode=mode)
    (2.0 * loss).backward(retain_graph=True)
    gH1, gW1 = H.grad.clone(), W.grad.clone()
    H.grad, W.grad = None, None
    (-0.5 * loss).backward()
    torch.cuda.synchronize()
    check(f"{mode}, first backward (g = 2)", float(loss.item()), f64(gH1), f64(gW1), ref, g=2.0)
    check(f"{mode}, second backward (g = -0.5)", float(loss.item()), f64(H.grad), f64(W.grad), ref, g=-0.5)


def test_autograd_without_gradients_runs_the_forward_only(problem):
    """Neither input requires a gradient: the loss alone, no gradient buffers
    (the peak allocation stays far below one grad_W)."""
    x, ref = problem
    dev = upload(x)
    ign = torch.from_numpy(x.ignore).cuda()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    loss = topk_kl_loss(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], ign, temperature=1.5, chunk=CHUNK)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    grad_w_bytes = x.V * x.d * 4
    say(f"  no-grad call: loss rel {loss_rel(float(loss.item()), ref['loss']):.2e}, "
        f"peak above inputs {extra} B (one fp32 grad_W: {grad_w_bytes} B)")
    assert not loss.requires_grad
    assert loss_rel(float(loss.item()), ref["loss"]) <= BF16_TOL["loss"]
    assert extra < grad_w_bytes // 4
    # only H requires a gradient: W.grad stays None, H.grad is the oracle's
    H = dev["H"].clone().requires_grad_(True)
    loss = topk_kl_loss(H, dev["W"], dev["topk_idx"], dev["topk_logit"], ign, temperature=1.5, chunk=CHUNK)
    loss.backward()
    torch.cuda.synchronize()
    assert rel_maxabs(f64(H.grad), ref["grad_H"]) <= BF16_TOL["grad"]


def test_scale_grads_into_fresh_outputs(problem):
    """Out of place: the kept fp32 gradients are untouched, out_H = g grad_H,
    and a bf16 out_W is g grad_W rounded to nearest even."""
    x, ref = problem
    dev = upload(x)
    ign = torch.from_numpy(x.ignore).cuda()
    _, gH, gW, _, _ = B.kd_topk_kl_fused(dev["H"], dev["W"], dev["topk_idx"], dev["topk_logit"], ign,
                                         temperature=1.5, chunk=CHUNK)
    gH0, gW0 = gH.clone(), gW.clone()
    g = torch.tensor([-1.75], device="cuda")
    oH = torch.empty_like(gH)
    oW = torch.empty(gW.shape, dtype=torch.bfloat16, device="cuda")
    B.kd_topk_kl_scale_grads(g, gH, gW, out_H=oH, out_W=oW)
    oW32 = torch.empty_like(gW)
    B.kd_topk_kl_scale_grads(g, grad_W=gW, out_W=oW32)
    torch.cuda.synchronize()
    assert torch.equal(gH, gH0) and torch.equal(gW, gW0)
    assert torch.equal(oW, (gW0 * -1.75).to(torch.bfloat16))     # fp32 product, then one rounding
    assert torch.equal(oW32, gW0 * -1.75)
    assert torch.equal(oH, (gH0.float() * -1.75).to(torch.bfloat16))
    eH = rel_maxabs(f64(oH), -1.75 * ref["grad_H"])
    eW = rel_maxabs(f64(oW), -1.75 * ref["grad_W"])
    say(f"  scaled into fresh outputs, g = -1.75: grad_H {eH:.2e}  grad_W (bf16) {eW:.2e}")
    assert eH <= BF16_TOL["grad"] and eW <= BF16_TOL["grad"]
