"""Build libqsa.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_qsa_amd.build

All HIP code is compiled with packed-FP32 VALU instructions disabled
(-target-feature -packed-fp32-ops): the kernels never need them.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqsa.so")
PROBE_SRC = os.path.join(PKG, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")   # the benchmark's stream-read ceiling, not the QSA ABI
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the QSA library needs ROCm to build")
    return exe


def _compile(srcs, out: str, verbose: bool) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC, "-o", tmp] + list(srcs)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr.strip():
        # the host pass reports the device-only target feature as unknown; harmless
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build libqsa.so and the benchmark's stream-read probe library."""
    _compile(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), LIB, verbose)
    _compile([PROBE_SRC], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
