"""The library's host code (argument validation, workspace layout, launch
set-up, status strings) built with AddressSanitizer and driven through every
host-side ABI check on the CPU: any out-of-bounds access, use after free or
similar error in that layer aborts the driver with a sanitizer report."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_host_layer_under_address_sanitizer():
    from block_sparse_attention_qsa_amd import build
    lib = build.build_asan()
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    r = subprocess.run([sys.executable, os.path.join(HERE, "abi_asan_driver.py"), lib], env=env,
                       capture_output=True, text=True, timeout=600)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ASAN_DRIVER_OK" in r.stdout
