"""The C-ABI boundary from plain C: tests/c/abi_check.c is compiled as C99
with gcc against include/qsa.h (no C++, no PyTorch), linked to libqsa.so and
run; it calls only entry points that need no GPU (version, status strings,
workspace sizing, argument checks that return before anything is
enqueued)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_sparse_attention_qsa_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c99_program_against_the_header(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = os.path.join(PKG, "libqsa.so")
    if not os.path.exists(lib):
        pytest.fail(f"{lib} is not built; run the package build")
    exe = str(tmp_path / "abi_check")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
           "-L", PKG, "-lqsa", f"-Wl,-rpath,{PKG}", "-L", os.path.join(ROCM, "lib"),
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi_check: ok" in run.stdout
