"""Build the HIP library ``libkdtopk.so`` for gfx950 with hipcc (in-tree), and
the MFMA-rate probe ``libkdprobe.so`` that ``bench.py --mfma-ceiling`` runs."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "kd_topk_kl.hip")
LIB = os.path.join(PKG, "libkdtopk.so")
PROBE_SRC = os.path.join(PKG, "csrc", "kd_mfma_ceiling.hip")
PROBE_LIB = os.path.join(PKG, "libkdprobe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def _hipcc(src: str, lib: str, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the loss library and the MFMA-rate probe; returns the loss library's path."""
    _hipcc(PROBE_SRC, PROBE_LIB, verbose)
    return _hipcc(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
