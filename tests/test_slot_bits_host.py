"""The select kernel's per-lane slot bit sets, checked on the host: the header
the kernel includes is compiled with g++ and run for 1, 64, 65 and 128 slots
(the 128-slot form once kept its bits in a single 64-bit word, where shifts of
64 and more are undefined)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_36_amd", "csrc")


def test_slot_bits_indexing(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "slot_bits_check"
    src = os.path.join(ROOT, "tests", "host", "slot_bits_check.cpp")
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-fsanitize=undefined",
                    "-fno-sanitize-recover=undefined", "-I", CSRC, src, "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    for spl in (1, 64, 65, 128):
        assert f"SPL={spl} words={(spl + 63) // 64} mismatches=0" in r.stdout
