"""The host-side C ABI (planner, metadata validator, predictor, online
calibration, batch former, split point) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: tests/sanitize builds those sources
with the GPU side stubbed out, runs a seeded fuzz driver over them, and the
host ABI tests run again against that build (the sanitizer runtime is
preloaded into a child Python). No GPU is used."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(SAN, "_build")


def asan_runtime():
    try:
        r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                           text=True, timeout=60)
    except OSError:
        return None
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def built():
    if shutil.which("make") is None or asan_runtime() is None:
        pytest.skip("needs make and g++ with AddressSanitizer")
    r = subprocess.run(["make", "-C", SAN, "-j8"], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return BUILD


def sanitizer_env(**extra):
    env = dict(os.environ)
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra)
    return env


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_fuzz_is_clean(built, seed):
    r = subprocess.run([os.path.join(built, "host_fuzz"), str(seed), "2000"],
                       capture_output=True, text=True, timeout=600,
                       env=sanitizer_env(ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-6000:]
    assert "checks passed" in r.stdout


def test_host_abi_tests_under_sanitizers(built):
    """tests/test_abi_host.py (planner, validator, predictor bit-exactness,
    calibration, scheduler, split point, NULL checks) against the sanitized
    build; leak checking is off because the Python interpreter itself is
    not built with the sanitizer."""
    env = sanitizer_env(CPA_LIBRARY=os.path.join(built, "libcpa_host_san.so"),
                        LD_PRELOAD=asan_runtime(),
                        ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi_host.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=900, env=env)
    out = r.stdout[-4000:] + r.stderr[-6000:]
    assert r.returncode == 0, out
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, out
    assert " passed" in r.stdout, out


def test_host_entry_points_under_thread_sanitizer():
    """tests/sanitize/host_threads.cpp under ThreadSanitizer: eight threads
    create, inspect, upload (to their own and to one shared workspace, which
    exercises the process-wide workspace registry) and destroy plans, hit
    refusals, and run the predictor, the calibration and the batch former;
    any data race fails the run."""
    if shutil.which("make") is None or not tsan_available():
        pytest.skip("needs make and g++ with ThreadSanitizer")
    r = subprocess.run(["make", "-C", SAN, "-j8", "tsan"], capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 second_deadlock_stack=1")
    r = subprocess.run([os.path.join(SAN, "_build_tsan", "host_threads")], capture_output=True,
                       text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-6000:]
    assert "host threads ok" in r.stdout


def tsan_available():
    try:
        r = subprocess.run(["g++", "-print-file-name=libtsan.so"], capture_output=True,
                           text=True, timeout=60)
    except OSError:
        return False
    path = r.stdout.strip()
    return os.path.isabs(path) and os.path.exists(path)
