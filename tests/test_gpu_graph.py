"""The fused entries captured in a HIP graph (torch.cuda.graph) and replayed.

The library enqueues only kernel launches on the caller's stream (no memset,
copy, allocation or synchronisation), so a caller can capture a whole fused
call.  Each graph is replayed several times with the program's own eager work
and device synchronisations between the replays; the outputs are set to NaN
before every replay, and every replay must reproduce the eager call bit for
bit, also after new input values are copied into the captured input buffers
(the graph reads its inputs at replay time).  Checked for the no-allocation
entry (its static scratch) and for the fused entry with a caller workspace.
"""
import numpy as np
import pytest
import torch

from chunked_top_kl_head_amd import binding as B
from chunked_top_kl_head_amd import synth

from .gpu_util import upload

pytestmark = pytest.mark.gpu

T, D, V, K, CHUNK = 700, 320, 5000, 50, 256


def say(*a):
    print(*a, flush=True)


def _outputs(dev):
    return dict(loss=torch.empty(1, dtype=torch.float32, device=dev),
                grad_H=torch.empty((T, D), dtype=torch.bfloat16, device=dev),
                grad_W=torch.empty((V, D), dtype=torch.float32, device=dev),
                lse=torch.empty(T, dtype=torch.float32, device=dev),
                row_loss=torch.empty(T, dtype=torch.float32, device=dev))


def _call(entry, d_in, out, ws):
    if entry == "noalloc":
        B.kd_topk_kl_fused_noalloc(d_in["H"], d_in["W"], d_in["topk_idx"], d_in["topk_logit"], d_in["ignore"],
                                   loss=out["loss"], grad_H=out["grad_H"], grad_W=out["grad_W"], lse=out["lse"],
                                   row_loss=out["row_loss"], chunk=CHUNK)
    else:
        loss, gH, gW, lse, rl = B.kd_topk_kl_fused(d_in["H"], d_in["W"], d_in["topk_idx"], d_in["topk_logit"],
                                                   d_in["ignore"], chunk=CHUNK, workspace=ws, grad_H=out["grad_H"],
                                                   grad_W=out["grad_W"], loss=out["loss"], want_lse=True,
                                                   want_row_loss=True)
        out["lse"].copy_(lse)
        out["row_loss"].copy_(rl)


def _same(a, b):
    return all(torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k].view(torch.int32),
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k].view(torch.int32))
               for k in a)


@pytest.mark.parametrize("entry", ["noalloc", "fused"])
def test_fused_call_in_a_graph(entry):
    dev = torch.device("cuda")
    say(f"entry {entry}: T={T} d={D} V={V} K={K} chunk={CHUNK}")
    x1 = synth.make_inputs(T, D, V, K, tau=1.0, dtype="bf16", seed=141, mask=("random", 0.1))
    x2 = synth.make_inputs(T, D, V, K, tau=1.0, dtype="bf16", seed=142, mask=("random", 0.1))
    in1, in2 = upload(x1), upload(x2)
    # the captured input buffers (x1's ignore mask has kept and ignored rows)
    d_in = {k: (v.clone() if v is not None else None) for k, v in in1.items()}
    ws = None
    if entry == "fused":
        prob = B.problem(T, D, V, K, 1.0, torch.bfloat16, CHUNK)
        ws = torch.empty(B.workspace_size(prob, B.KD_OP_FUSED), dtype=torch.uint8, device=dev)

    # eager references for both input sets
    assert in1["ignore"] is not None and in2["ignore"] is not None
    refs = []
    for src in (in1, in2):
        out = _outputs(dev)
        _call(entry, src, out, ws)
        torch.cuda.synchronize()
        refs.append({k: v.clone() for k, v in out.items()})

    out = _outputs(dev)
    _call(entry, d_in, out, ws)            # warm-up on the capture buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(entry, d_in, out, ws)
    torch.cuda.synchronize()

    side = torch.randn(1 << 20, device=dev)
    for rep in range(3):
        for v in out.values():
            v.fill_(float("nan"))
        side.mul_(1.0001).add_(0.5)        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, refs[0]), f"replay {rep} differs from the eager call"
        say(f"  replay {rep}: bitwise equal to the eager call")

    # new input values in the captured buffers: the replay must follow them
    for k in ("H", "W", "topk_idx", "topk_logit", "ignore"):
        d_in[k].copy_(in2[k])
    torch.cuda.synchronize()
    for rep in range(2):
        for v in out.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(out, refs[1]), f"replay {rep} on new inputs differs from the eager call"
        say(f"  replay {rep} on new inputs: bitwise equal to the eager call")
    assert np.isfinite(float(out["loss"].item()))
