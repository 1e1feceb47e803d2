"""The host plan builder under AddressSanitizer and UBSan.

plan.cpp is plain C++ (no HIP), so it is compiled here with g++ together with
plan_fuzz.cpp, which builds plans for random and degenerate tries at every
conv width and compares every table with a brute-force walk over the trie's
token paths, then feeds invalid tries and arguments.  Any out-of-bounds
access, overflow or mismatch fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_tree_packed_plan_amd", "csrc")


def test_plan_builder_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "plan_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "plan_fuzz.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if build.returncode != 0 and "asan" in build.stderr.lower() and "cannot find" in build.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "all tables match" in run.stdout
