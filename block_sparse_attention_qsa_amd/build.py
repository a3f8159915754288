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
DEBUG_LIB = os.path.join(PKG, "libqsa_debug.so")   # same ABI, device-side precondition checks
PROBE_SRC = os.path.join(PKG, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")   # the benchmark's stream-read ceiling, not the QSA ABI
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the QSA library needs ROCm to build")
    return exe


def _command(srcs, out: str, defines=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC] + [f"-D{d}" for d in defines] + ["-o", out] + list(srcs)


def _finish(proc, cmd, tmp: str, out: str, verbose: bool) -> str:
    stdout, stderr = proc.communicate()
    if proc.returncode != 0:
        sys.stderr.write(stdout + stderr)
        raise RuntimeError(f"hipcc failed with status {proc.returncode}: {' '.join(cmd)}")
    if verbose and stderr.strip():
        # the host pass reports the device-only target feature as unknown; harmless
        lines = [l for l in stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build libqsa.so, its debug twin libqsa_debug.so (QSA_DEBUG_CHECKS) and
    the benchmark's stream-read probe library, the three hipcc runs at once."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = [(srcs, LIB, ()), (srcs, DEBUG_LIB, ("QSA_DEBUG_CHECKS",)), ([PROBE_SRC], PROBE_LIB, ())]
    running = []
    for sources, out, defines in jobs:
        tmp = out + f".tmp{os.getpid()}"
        cmd = _command(sources, tmp, defines)
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True),
                        cmd, tmp, out))
    for proc, cmd, tmp, out in running:
        _finish(proc, cmd, tmp, out, verbose)
    return LIB


ASAN_LIB = os.path.join(PKG, "_build", "libqsa_asan.so")   # host code under AddressSanitizer (CPU tests)


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (to preload into a
    process that loads ASAN_LIB)."""
    llvm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no shared AddressSanitizer runtime found next to hipcc")
    return hits[-1]


def build_asan(verbose: bool = False) -> str:
    """Build the library with its host code (the ABI layer: validation,
    workspace layout, launch set-up) under AddressSanitizer; device code is
    built as usual."""
    os.makedirs(os.path.dirname(ASAN_LIB), exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = ASAN_LIB + f".tmp{os.getpid()}"
    cmd = _command(srcs, tmp) + ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                                 "-shared-libsan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    return _finish(proc, cmd, tmp, ASAN_LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
