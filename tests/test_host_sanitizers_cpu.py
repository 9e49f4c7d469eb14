"""The library's host code (offline preparation, input-aware preparation,
plan packing, size/offset queries and their error paths) built from source
with AddressSanitizer + UndefinedBehaviorSanitizer, and with
ThreadSanitizer for the worker pool, then driven by tests/native/host_sanitize.cpp
on small specs of every structure.  CPU only: the host sources hold no HIP."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "input_adaptive_rank_amd", "csrc")
SOURCES = [os.path.join(CSRC, "prepare.cpp"), os.path.join(CSRC, "host_linalg.cpp"),
           os.path.join(ROOT, "tests", "native", "host_sanitize.cpp")]
BASE = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-mavx2", "-mfma",
        "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def _build_and_run(tmp_path, flags, env, args=()):
    exe = str(tmp_path / "host_sanitize")
    b = subprocess.run(BASE + flags + SOURCES + ["-o", exe, "-lpthread"], capture_output=True, text=True)
    if b.returncode != 0 and "sanitize" in b.stderr and "cannot find" in b.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=600,
                       env={**os.environ, **env})
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "all checks passed" in r.stdout
    for marker in ("AddressSanitizer", "LeakSanitizer", "runtime error", "ThreadSanitizer"):
        assert marker not in report, report[-6000:]


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                   {"ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"})


def test_host_worker_pool_under_thread_sanitizer(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"}, args=("small",))
