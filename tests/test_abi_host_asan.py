"""The C ABI's host layer under AddressSanitizer (CPU only, no device calls).

The argument validation and launch planning of the library (w8inv_api.hip) are built with ASan on
their host side (invariant_quantized_decode_amd/build.py, build_host_asan) and linked with the
product's other objects; test_abi_cpu.py then runs in a child process that preloads the ASan
runtime and routes the binding to that library.  Every rejected argument, size query and
kernel-name query of that module goes through instrumented code, so an out-of-bounds access, a
use after free or a bad free in the host layer fails here.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_w8inv_build", os.path.join(ROOT, "invariant_quantized_decode_amd",
                                                                                 "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


CHILD = """
import sys
import pytest
import invariant_quantized_decode_amd as w8
w8._lib = w8._load(sys.argv[1])
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", sys.argv[2]]))
"""


def test_abi_validation_is_clean_under_host_asan():
    b = _build_module()
    runtime = b.asan_runtime()
    if not runtime:
        pytest.skip("no ASan runtime in the ROCm toolchain")
    lib = b.build_host_asan()
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0:exitcode=86")
    r = subprocess.run([sys.executable, "-c", CHILD, lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = (r.stdout + r.stderr)[-4000:]
    assert "AddressSanitizer" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
