"""The host-side C ABI tests (tests/test_abi_host.py) against a copy of librehyat.so whose
host code (api.cpp: argument checks, workspace layout, overlap checks, launch sequences) is
built with AddressSanitizer and UndefinedBehaviorSanitizer, run in a child process with the
sanitizer runtime preloaded. No kernel is launched (every call there fails validation
first), so this runs without a GPU. A memory error or undefined behaviour in the host code
ends the child with the sanitizer's report.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _toolchain():
    from hybrid_softmax_linear_amd import build as b
    try:
        b.hipcc()
        return b, b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))


def test_abi_host_tests_under_asan_and_ubsan(tmp_path):
    b, runtime = _toolchain()
    lib = b.build_host_sanitized(str(tmp_path / "librehyat_hostsan.so"))
    env = dict(os.environ)
    env.update({"LD_PRELOAD": runtime, "REHYAT_LIBRARY": lib,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert res.returncode == 0, out[-3000:]
    assert " passed" in out
