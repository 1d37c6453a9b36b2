"""The library's host-only C++ (packer, unpacker, region table, bit
allocation, baseline packers) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and run on seeded inputs and edge cases by
tests/san_driver.cpp: any out-of-bounds access, leak or undefined behaviour
aborts the run.  CPU only."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "tenant_rank_serving_amd", "csrc")
HOST_SOURCES = ["pack.cpp", "alloc.cpp", "pack_baselines.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-static-libasan"]


def test_host_code_under_sanitizers():
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "san_driver")
        cmd = (["g++", "-std=c++17", "-O1", "-g", "-Wall", "-I", os.path.join(ROOT, "include")] + SAN +
               [os.path.join(HERE, "san_driver.cpp")] + [os.path.join(CSRC, f) for f in HOST_SOURCES] +
               ["-o", exe])
        b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert b.returncode == 0, b.stdout
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
        assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout[-4000:]
