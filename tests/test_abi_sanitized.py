"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of the library whose api.cpp (argument validation and launch
set-up) is compiled with -fsanitize=address,undefined, then runs the CPU ABI
tests (tests/test_abi.py: every call there is rejected on the host, so no
kernel is launched and no GPU is needed) in a child process that preloads
the sanitizer runtime.  Any sanitizer report aborts the child and fails this
test."""

import os
import shutil
import subprocess
import sys

import pytest

from attention_fa2_tiles_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_rejections_under_host_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    try:
        path = build.build_host_sanitized(str(tmp_path))
    except FileNotFoundError as e:
        pytest.skip(str(e))
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.exists(asan), asan
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, FA2TILES_ABI_TEST_LIB=path,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
