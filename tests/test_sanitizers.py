"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU, gcc and g++): the
oracle's every form on inputs in buffers of exactly their length (a read past a message's
last byte, a leak or undefined behaviour ends the run), and the batch planner on random
and edge-case batches with a check of each plan's layout. The drivers are in
tests/sanitize/."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _build_and_run(cmd, exe, timeout=300):
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=timeout)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, timeout=timeout, env=env)


def test_sanitizers_catch_planted_errors(tmp_path):
    # the instrumented builds are live: AddressSanitizer stops a one-byte read past a heap
    # buffer, UndefinedBehaviorSanitizer a signed overflow
    over = tmp_path / "over.c"
    over.write_text("#include <stdlib.h>\nint main(void) { volatile unsigned char *p = malloc(16);\n"
                    "  int v = p[16]; free((void *)p); return v == 1234; }\n")
    r = _build_and_run(["gcc", "-O1", "-g", "-fsanitize=address", str(over), "-o", str(tmp_path / "over")],
                       str(tmp_path / "over"))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
    ub = tmp_path / "ub.c"
    ub.write_text("#include <limits.h>\nint main(void) { volatile int x = INT_MAX; return x + 1 == 0; }\n")
    r = _build_and_run(["gcc", *SAN, str(ub), "-o", str(tmp_path / "ub")], str(tmp_path / "ub"))
    assert r.returncode != 0 and "signed integer overflow" in r.stderr


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    r = _build_and_run(["gcc", "-std=c11", *SAN, "-pthread", os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                        os.path.join(ROOT, "oracle", "blake3_oracle.c"), "-o", exe], exe)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all forms agree" in r.stdout


def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_driver")
    csrc = os.path.join(ROOT, "blake3_merkle_tree_amd", "csrc")
    r = _build_and_run(["g++", "-std=c++17", *SAN, "-I", csrc, os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
                        os.path.join(csrc, "b3_plan.cpp"), "-o", exe], exe)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "every plan well formed" in r.stdout
