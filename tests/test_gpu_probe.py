"""The MFMA-rate probe (libkdprobe.so) that bench.py --mfma-ceiling times.

Mode 3 gives every lane the same operands: A fragment elements
a = (1, 1, 0.5, 0.5, 0.25, 0.25, 0.5, 1) and B fragment elements
b = (1, 0.5, 1, 0.25, 1, 1, 0.25, 0.5) (bf16, element j of a lane at k = 8 (lane / 32) + j).
Each step then adds sum over k < 16 of a[k mod 8] b[k mod 8] = 2 x 3.25 = 6.5 to every
one of a wave's 8 x 16 accumulator elements per lane, exactly in fp32, so a thread's
sum of its accumulators after `iters` steps is 128 x 6.5 x iters = 832 iters: proof that
every MFMA the FLOP count assumes was executed.  The other modes must give finite sums.
"""
import ctypes

import pytest
import torch

from chunked_top_kl_head_amd import build as hip_build

pytestmark = pytest.mark.gpu


def _probe():
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    f = lib.kd_probe_mfma_launch
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return f


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_probe_executes_every_mfma(mode):
    f = _probe()
    wgs, iters = 300, 1000
    dev = torch.device("cuda:0")
    sink = torch.full((wgs * 512,), float("nan"), dtype=torch.float32, device=dev)
    cycles = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    print(f"probe mode {mode}: {wgs} workgroups, {iters} steps", flush=True)
    rc = f(mode, wgs, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(cycles.data_ptr()),
           ctypes.c_void_p(stream.cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    s = sink.cpu()
    c = cycles.view(wgs, 2).cpu()
    assert bool((c > 0).all()), "every workgroup records its shader cycles and real-time ticks"
    if mode == 3:
        assert bool((s == 832.0 * iters).all()), f"sums {s.min().item()} .. {s.max().item()}"
    else:
        assert bool(torch.isfinite(s).all())
