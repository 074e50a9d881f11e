"""The C ABI checks of test_abi.py and test_abi_fuzz.py, run against the sanitized
build of the host layer: api.cpp compiled by g++ with AddressSanitizer and
UndefinedBehaviorSanitizer (every validation, sizing and error path the tests
drive), in a child process with the ASan runtime preloaded.  CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if not shutil.which("g++"):
        return None
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_env():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("g++ with libasan is not available")
    sys.path.insert(0, ROOT)
    from block_sparse_attention_36_amd import build
    lib = build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, BSA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env, lib


def test_sanitized_library_is_the_one_loaded(sanitized_env):
    env, lib = sanitized_env
    code = ("import block_sparse_attention_36_amd as b; b.load_library(); "
            "print(open('/proc/self/maps').read())")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 0, out.stderr[-2000:]
    assert os.path.basename(lib) in out.stdout and "libasan" in out.stdout


def test_abi_checks_pass_under_asan_and_ubsan(sanitized_env):
    env, _ = sanitized_env
    out = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"),
                          os.path.join(ROOT, "tests", "test_abi_fuzz.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, (out.stdout[-3000:] + out.stderr[-3000:])
    assert "passed" in out.stdout and "ERROR: AddressSanitizer" not in out.stderr
    assert "runtime error" not in out.stderr
