"""The C ABI's argument checks under AddressSanitizer (CPU only): api.cpp is
rebuilt by g++ with the sanitizer (build.build_asan) and tests/test_abi.py runs
against that library in a child process with the sanitizer runtime preloaded.
Any invalid read or write in the validation and dispatch code then aborts the
child with a sanitizer report."""

import os
import shutil
import subprocess
import sys

import pytest

from exact_tiled_attention_11_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++ with libasan")
def test_abi_checks_under_address_sanitizer():
    lib = build.build_asan()
    rt = build.asan_runtime()
    assert os.path.isabs(rt) and os.path.exists(rt), rt
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_report_load" in nm.stdout, "api.cpp is not instrumented"
    env = dict(os.environ, FA355_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr
