"""Runs the host-side ABI checks of abi_cases.py against the library build
whose host code is compiled with AddressSanitizer.  Started by
test_abi_asan.py in a process that preloads the sanitizer runtime; imports
neither torch nor the package (its ctypes declarations are loaded by path)."""
import importlib.util
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _load(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


abi = _load("qsa_abi_decls", os.path.join(ROOT, "block_sparse_attention_qsa_amd", "_abi.py"))
cases = _load("abi_cases", os.path.join(HERE, "abi_cases.py"))
lib = abi.load(sys.argv[1])
for _ in range(3):            # repeated, so that any heap misuse in the host layer gets a chance to show
    cases.run_all(lib, abi.CBatch)
print("ASAN_DRIVER_OK", flush=True)
