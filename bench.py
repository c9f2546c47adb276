#!/usr/bin/env python3
"""Benchmark of the fused chunked top-K KL loss (forward + backward) on one MI355X.

One step = one call of the fused entry point over every position of the
workload (logits GEMM, row kernel, grad_H GEMM and grad_W GEMM for each chunk),
with inputs, outputs and workspace resident in HBM before the timed region.
Prints one JSON line.  The default workload is the GPT-OSS-20B-like shape
(T = 32768 positions, d = 2880, V = 201088, K = 100, bf16).

Timing: W untimed warmup steps, then K steps bracketed by device
synchronisation; per-kernel launch durations come from HIP events that the
library records around each launch of every stage on the launch stream
(kd_topk_kl_set_stage_events), over the same timed steps.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3  # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "fwd+bwd tokens/s of fused top-K KL loss; MFMA util % of bf16 peak; peak HBM GiB"
KERNEL_SOURCES = ("kd_common.hpp", "kd_gemm.hpp", "kd_gemm_dtl.hpp", "kd_kernels.hpp", "kd_topk_select.hpp",
                  "kd_topk_kl.hip")


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed (string and
    character literals kept), so that comment edits leave the hash alone."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(sources: dict | None = None) -> str:
    """Hash of the kernel sources' code (comments and whitespace excluded);
    ``sources`` maps file name to text (default: the files in csrc/)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        if sources is None:
            with open(os.path.join(ROOT, "chunked_top_kl_head_amd", "csrc", f), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = sources[f]
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw HIP events from the runtime the process already loaded (torch's)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            rc = self.rt.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = e.value
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, arr):
        for e in arr:
            self.rt.hipEventDestroy(ctypes.c_void_p(e))


def cpu_baseline(x, rows: int) -> dict:
    """The fp64 oracle on the first `rows` positions of the same workload (fwd + both grads)."""
    from oracle import kd_oracle

    sel = slice(0, rows)
    t0 = time.perf_counter()
    kd_oracle.full(x.H[sel], x.W, x.topk_idx[sel], x.topk_logit[sel], x.ignore[sel], tau=x.tau)
    dt = time.perf_counter() - t0
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": rows / dt, "unit": "tokens/s", "cores": kd_oracle.num_threads(), "kind": "oracle",
            "sample": f"first {rows} positions of the workload, full vocabulary, fwd + grad_H + grad_W, "
                      f"fp64, {dt:.1f} s", "cpu": cpu}


def bench_select(args) -> int:
    """The teacher top-K cache producer (kd_topk_select) on the teacher logits of
    the GPT-OSS-like workload: T = 32768 rows of V = 201088 bf16 logits, K = 100.
    One step = one call over all rows; prints one JSON line."""
    import numpy as np
    import torch

    from chunked_top_kl_head_amd import binding as B

    T, V, K = 32768, 201088, 100
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(20261203)
    logits = (torch.randn(T, V, device=dev, generator=g) * 3).to(torch.bfloat16)
    for _ in range(args.warmup):
        B.kd_topk_select(logits, K)
    ev = HipEvents()
    whole = ev.create(2)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    ev.rt.hipEventRecord(ctypes.c_void_p(whole[0]), ctypes.c_void_p(stream.cuda_stream))
    for _ in range(args.steps):
        idx, val = B.kd_topk_select(logits, K)
    ev.rt.hipEventRecord(ctypes.c_void_p(whole[1]), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(whole[0], whole[1]) / args.steps
    ev.destroy(whole)
    algo_bytes = T * V * 2 + T * K * 8           # read the logits once, write ids + fp32 logits
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "teacher top-K cache rows/s (per-row top-100 of bf16 logits)",
        "value": round(T / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (3 * N(0,1) logits)",
        "config": {"workload": f"topk_select: T={T} V={V} K={K} bf16"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "topk_select"},
    }
    if not args.no_cpu_baseline:
        from oracle.topk_select import topk_select

        rows = min(args.cpu_rows, T)
        sub = logits[:rows].float().cpu().numpy()
        t0 = time.perf_counter()
        topk_select(sub, K)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": rows / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {rows} rows, numpy lexsort per row, {dt:.1f} s"}
    del np
    print(json.dumps(out), flush=True)
    return 0


def bench_mfma_ceiling(args) -> int:
    """The part's sustained bf16 MFMA rate with no global memory traffic
    (libkdprobe.so): 256 workgroups of 8 waves, each wave running the engine's
    8-MFMA step on constant random operands (mode 0), on operand bits that change
    every step in registers (mode 1), on random bf16 fragments read from LDS in
    the engine's pattern (mode 2) and on constant operands of few set bits
    (mode 3).  For each mode: the launch time (HIP events), the
    shader clock the launch ran at (per-workgroup s_memtime cycles over
    s_memrealtime 100 MHz ticks) and the MFMA TFLOP/s.  Prints one JSON line."""
    import torch

    from chunked_top_kl_head_amd import build as hip_build

    path = hip_build.PROBE_LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.kd_probe_mfma_launch.restype = ctypes.c_int
    lib.kd_probe_mfma_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    wgs, iters = 256, 200000
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    cycles = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    flop = wgs * 8 * iters * 8 * 32768.0
    names = {0: "constant random operands", 1: "operands changing every step (registers)",
             2: "random bf16 operands from LDS", 3: "constant operands of few set bits"}
    modes = []
    for mode in (0, 1, 2, 3):
        runs = []
        for rep in range(max(1, args.warmup) + max(1, args.steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.kd_probe_mfma_launch(mode, wgs, iters, ctypes.c_void_p(sink.data_ptr()),
                                          ctypes.c_void_p(cycles.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"kd_probe_mfma_launch failed: hipError {rc}")
            e1.record(stream)
            torch.cuda.synchronize()
            if rep < max(1, args.warmup):
                continue
            ms = e0.elapsed_time(e1)
            c = cycles.view(wgs, 2).double().sum(dim=0).tolist()
            ghz = c[0] / c[1] * 0.1
            runs.append((ms, flop / (ms * 1e-3) / 1e12, ghz))
            print(f"mode {mode}: {ms:.2f} ms {runs[-1][1]:.1f} TFLOP/s at {ghz:.3f} GHz", file=sys.stderr, flush=True)
        ms = sorted(r[0] for r in runs)[len(runs) // 2]
        best = min(runs, key=lambda r: abs(r[0] - ms))
        modes.append({"mode": mode, "operands": names[mode], "ms": round(best[0], 3),
                      "tflops": round(best[1], 1), "clock_ghz": round(best[2], 3),
                      "frac_of_nominal": round(best[1] / PEAK_BF16_TFLOPS, 4),
                      "busy_at_clock": round(best[1] / (PEAK_BF16_TFLOPS * best[2] / 2.4), 4)})
    out = {"metric": "sustained bf16 MFMA rate, no memory traffic", "unit": "TFLOP/s", "n_gpus": 1,
           "peak_nominal": PEAK_BF16_TFLOPS, "nominal_clock_ghz": 2.4,
           "config": {"workload": f"mfma_ceiling: {wgs} workgroups x 8 waves, {iters} steps of 8 "
                                  "v_mfma_f32_32x32x16_bf16 per wave"},
           "modes": modes}
    print(json.dumps(out), flush=True)
    return 0


def bench_teacher(args) -> int:
    """The cache producer from hidden states (kd_teacher_topk) with the
    workload's H [T, d] and W [V, d] standing in for the teacher's: per chunk a
    logits GEMM into fp32 and the per-row top-K.  One step = one call over all
    positions; prints one JSON line (dominant cost: the GEMM, 2 T d V FLOP)."""
    import numpy as np
    import torch

    from chunked_top_kl_head_amd import binding as B
    from chunked_top_kl_head_amd import synth

    x = synth.workload_inputs(args.workload)
    dev = torch.device("cuda:0")
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(x.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H = torch.from_numpy(x.H).to(dev)
        W = torch.from_numpy(x.W).to(dev)
    T, d, V, K = x.T, x.d, x.V, 100
    chunk = args.chunk or 4096
    prob = B.KdTeacherProblem(T, d, V, K, chunk, B.KD_BF16 if x.dtype == "bf16" else B.KD_F32, 0)
    lib = B.load_library()
    n = ctypes.c_size_t(0)
    B._check("kd_teacher_topk_workspace_size", lib.kd_teacher_topk_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    ws = torch.empty(int(n.value), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        B.kd_teacher_topk(H, W, K, chunk=chunk, workspace=ws)
    ev = HipEvents()
    whole = ev.create(2)
    stream = torch.cuda.current_stream()
    torch.cuda.reset_peak_memory_stats()
    torch.cuda.synchronize()
    ev.rt.hipEventRecord(ctypes.c_void_p(whole[0]), ctypes.c_void_p(stream.cuda_stream))
    for _ in range(args.steps):
        B.kd_teacher_topk(H, W, K, chunk=chunk, workspace=ws)
    ev.rt.hipEventRecord(ctypes.c_void_p(whole[1]), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(whole[0], whole[1]) / args.steps
    ev.destroy(whole)
    tflops = 2.0 * T * d * V / (ms * 1e-3) / 1e12
    peak = 2500.0 if x.dtype == "bf16" else 157.3
    out = {
        "metric": "teacher top-K cache rows/s from hidden states (top-100 of H W^T per position)",
        "value": round(T / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": x.dtype, "data": "synthetic (seeded H, W)",
        "config": {"workload": f"teacher_topk: T={T} d={d} V={V} K={K} {x.dtype}", "chunk": chunk},
        "tflops": round(tflops, 2), "peak_hbm_gib": round(torch.cuda.max_memory_allocated() / 2**30, 3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None, "kernel": "whole call"},
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_vendor_gemm(args) -> int:
    """Yardstick for the engine's per-launch rates: the vendor BLAS (hipBLASLt,
    through torch.matmul) on the three contraction shapes of one full chunk of
    the workload, with bf16 outputs and no epilogue work (logits H_c W^T, grad_H
    G_c W, grad_W G_c^T H_c).  Operands are seeded random bf16 of the workload's
    scales.  Prints one JSON line."""
    import torch

    from chunked_top_kl_head_amd import synth

    wl = synth.WORKLOADS[args.workload]
    C = min(args.chunk or wl.chunk, wl.T)
    d, V = wl.d, wl.V
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    W = (torch.randn(V, d, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    H = torch.randn(C, d, device=dev, generator=gen).to(torch.bfloat16)
    G = (torch.randn(C, V, device=dev, generator=gen) * 1e-3).to(torch.bfloat16)
    flop = 2.0 * C * d * V
    cases = [("logits", lambda: torch.matmul(H, W.t())),
             ("grad_H", lambda: torch.matmul(G, W)),
             ("grad_W", lambda: torch.matmul(G.t(), H))]
    stream = torch.cuda.current_stream()
    res = []
    for name, fn in cases:
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(max(1, args.steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        res.append({"gemm": name, "ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                    "frac": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
        print(f"{name}: {ms:.3f} ms {res[-1]['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    out = {"metric": "vendor BLAS (torch.matmul -> hipBLASLt) on the loss's contraction shapes, median launch",
           "unit": "TFLOP/s", "n_gpus": 1, "peak": PEAK_BF16_TFLOPS, "dtype": "bf16",
           "config": {"workload": f"{args.workload}: one chunk of {C} rows, d={d}, V={V}", "chunk": C},
           "gemms": res}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    from chunked_top_kl_head_amd import synth

    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gptoss20b", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--chunk", type=int, default=0, help="rows per chunk (0 = the workload's)")
    ap.add_argument("--mode", default="fused", choices=["fused", "split"],
                    help="fused entry, or forward followed by backward")
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--select", action="store_true",
                    help="benchmark the teacher top-K cache producer instead of the loss")
    ap.add_argument("--teacher", action="store_true",
                    help="benchmark the cache producer from hidden states (kd_teacher_topk): the workload's "
                         "H and W as the teacher's, K = 100")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="measure the part's sustained bf16 MFMA rate and clock with no memory traffic "
                         "(constant, changing and LDS-fed random operands)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the vendor BLAS (torch.matmul) on the three contraction shapes of one chunk, "
                         "plain bf16 outputs: a yardstick for the engine's per-launch rates")
    ap.add_argument("--copy-calibration-bytes", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many bytes (a kernel of known "
                         "traffic, used to scale the FETCH_SIZE/WRITE_SIZE counters of a profiling run)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs the loss on a single GPU; positions shard naturally across GPUs "
              "but no multi-GPU path is built. Run with --gpus 1.", file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    from chunked_top_kl_head_amd import binding as B

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.select:
        return bench_select(args)
    if args.teacher:
        return bench_teacher(args)
    if args.mfma_ceiling:
        return bench_mfma_ceiling(args)
    if args.vendor_gemm:
        return bench_vendor_gemm(args)
    wl = synth.WORKLOADS[args.workload]
    chunk = args.chunk or wl.chunk
    t_gen = time.perf_counter()
    x = synth.workload_inputs(args.workload)
    gen_s = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    if x.dtype == "bf16":
        H = torch.from_numpy(x.H_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(x.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        H = torch.from_numpy(x.H).to(dev)
        W = torch.from_numpy(x.W).to(dev)
    idx = torch.from_numpy(x.topk_idx).to(dev)
    lg = torch.from_numpy(x.topk_logit).to(dev)
    ig = torch.from_numpy(x.ignore).to(dev) if x.ignore.any() else None
    T, d, V, K = x.T, x.d, x.V, x.K

    prob = B.problem(T, d, V, K, x.tau, H.dtype, chunk)
    op = B.KD_OP_FUSED if args.mode == "fused" else B.KD_OP_BACKWARD
    ws_bytes = B.workspace_size(prob, op)
    if args.mode == "split":
        ws_bytes = max(ws_bytes, B.workspace_size(prob, B.KD_OP_FORWARD))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    gH = torch.empty_like(H)
    gW = torch.empty((V, d), dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)

    def step():
        if args.mode == "fused":
            B.kd_topk_kl_fused(H, W, idx, lg, ig, temperature=x.tau, chunk=chunk, workspace=ws,
                               grad_H=gH, grad_W=gW, loss=loss)
        else:
            l, s, _ = B.kd_topk_kl_forward(H, W, idx, lg, ig, temperature=x.tau, chunk=chunk, workspace=ws)
            B.kd_topk_kl_backward(H, W, idx, lg, s, ig, temperature=x.tau, chunk=chunk, workspace=ws,
                                  grad_H=gH, grad_W=gW)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-stage launch events over the timed steps
    lib = B.load_library()
    ev = HipEvents()
    nchunks = (T + chunk - 1) // chunk
    # launches per chunk and stage: the row kernel runs before and after the
    # logits GEMM in the forward and fused entries and once more in the split
    # backward; the split path runs the logits GEMM in both passes
    split = args.mode == "split"
    per_chunk = {B.KD_STAGE_LOGITS: 2 if split else 1, B.KD_STAGE_ROWS: 3 if split else 2,
                 B.KD_STAGE_GRAD_H: 1, B.KD_STAGE_GRAD_W: 1}
    expected = {st: args.steps * nchunks * n for st, n in per_chunk.items()}
    tables = []
    for st in range(4):
        cap = expected[st]
        b, e = ev.create(cap), ev.create(cap)
        cnt = ctypes.c_int(0)
        B._check("kd_topk_kl_set_stage_events", lib.kd_topk_kl_set_stage_events(st, b, e, cap, ctypes.byref(cnt)))
        tables.append((b, e, cnt))
    # one event before the first timed step and one after each step
    marks = ev.create(args.steps + 1)
    stream = torch.cuda.current_stream()
    torch.cuda.reset_peak_memory_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.rt.hipEventRecord(ctypes.c_void_p(marks[0]), ctypes.c_void_p(stream.cuda_stream))
    for i in range(args.steps):
        step()
        ev.rt.hipEventRecord(ctypes.c_void_p(marks[i + 1]), ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for st in range(4):
        lib.kd_topk_kl_set_stage_events(st, None, None, 0, None)
    peak_gib = torch.cuda.max_memory_allocated() / 2**30
    gpu_ms = ev.elapsed_ms(marks[0], marks[args.steps])
    ms_per_step = gpu_ms / args.steps
    step_ms = sorted(ev.elapsed_ms(marks[i], marks[i + 1]) for i in range(args.steps))

    # per-stage durations
    stages = {}
    rows_full = min(chunk, T)
    for st, (b, e, cnt) in enumerate(tables):
        n = cnt.value
        if n != expected[st]:
            raise RuntimeError(f"stage {B.STAGE_NAMES[st]}: {n} launches recorded, {expected[st]} expected")
        durs = [ev.elapsed_ms(b[i], e[i]) for i in range(n)]
        stages[B.STAGE_NAMES[st]] = dict(launches=n, avg_ms=(sum(durs) / n if n else 0.0),
                                         total_ms_per_step=sum(durs) / args.steps)
        ev.destroy(b)
        ev.destroy(e)
    ev.destroy(marks)
    dom = max(stages, key=lambda k: stages[k]["total_ms_per_step"])
    flops_step = 6.0 * T * d * V
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if x.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    # algorithmic work of one launch of the dominant stage: a full chunk of rows
    if dom in ("logits", "grad_H", "grad_W"):
        per_launch = 2.0 * rows_full * d * V
        achieved = per_launch / (stages[dom]["avg_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        # row kernel: reads and rewrites the chunk's G rows, reads the (max, sum)
        # partials (one per 128 ids) and the cached ids and logits
        V_pad = (V + 255) // 256 * 256
        per_launch = rows_full * (2.0 * 2 * V_pad + 8.0 * (V_pad // 128) + 8.0 * K)
        achieved = per_launch / (stages[dom]["avg_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["traffic"] = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tr = json.load(fh)
        ent = tr.get(args.workload, {}).get(dom)
        # the figures are per launch of the fused entry's kernels at one chunk size
        if (ent and ent.get("source_sha") == kernel_source_hash() and ent.get("chunk") == chunk
                and ent.get("mode", "fused") == args.mode):
            roof["traffic"] = ent["bytes_per_launch"]

    out = {
        "metric": METRIC,
        "value": round(T * args.steps / (gpu_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 3),
        "ms_per_step_min": round(step_ms[0], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic (seeded H, W, Zipf(1.1) top-K ids, 3*Gumbel teacher logits)",
        "config": {"workload": f"{wl.name}: T={T} d={d} V={V} K={K} tau={x.tau} {x.dtype}"
                               + (f" mask={wl.mask[0]}" if wl.mask else ""),
                   "chunk": chunk, "mode": args.mode, "positions": T, "kept": int(x.N),
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_util_pct": round(100.0 * tflops / peak, 2),
        "peak_hbm_gib": round(peak_gib, 3),
        "wall_s": round(wall, 3),
        "stages": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                   for k, v in stages.items()},
        "roofline": roof,
        "input_gen_s": round(gen_s, 1),
    }
    if args.copy_calibration_bytes > 0:
        src = torch.ones(args.copy_calibration_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = args.copy_calibration_bytes
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, min(args.cpu_rows, T))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
