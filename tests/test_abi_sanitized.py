"""The C ABI's CPU tests (tests/test_abi.py) once more against a host-sanitizer build of the library.

The host code (argument validation, workspace carving, the error paths, side-stream checks) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer; any out-of-bounds access, use after free or undefined
behaviour on those paths aborts the child process.  No GPU is used.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_dg_build_san", os.path.join(ROOT, "block_diffusion_decoding_step_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_tests_under_asan_and_ubsan():
    b = _build_module()
    lib = b.build_sanitized()
    rt = b.asan_runtime()
    assert os.path.exists(rt), rt
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "the host code is not instrumented"
    env = dict(os.environ, DG_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
