"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/planner_fuzz.cpp drives make_plan with seeded random problem
descriptions (small, ragged, aligned and large sizes, both dtypes, every cell
and regime, several device sizes) and checks the invariants the launch code
relies on; it is built here with g++ (host code only) and the sanitizers, and
must run clean.  CPU only.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "stacked_lstm_forward_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_fuzz_under_sanitizers(tmp_path):
    exe = str(tmp_path / "planner_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(ROOT, "tests", "native", "planner_fuzz.cpp"),
           os.path.join(CSRC, "lstm_plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in ("1", "20240601"):
        r = subprocess.run([exe, "20000", seed], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.startswith("ok:"), r.stdout
        assert "runtime error" not in r.stderr, r.stderr
