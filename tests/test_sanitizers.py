"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU): the
planner that derives the relations and exchange rounds (plan.cpp) and the C
oracle, each built with gcc/g++ and both sanitizers into a small driver that
exercises every shape and orientation, random relations, and cascades of
every type at odd sizes on one and several threads.  Any sanitizer report
ends the driver with a nonzero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(tmp_path, compiler, srcs, extra):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / "driver")
    r = subprocess.run([compiler] + SAN + srcs + extra + ["-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-4000:]
    return run.stdout


def test_planner_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "chip_fusion_amd", "csrc")
    out = _build_and_run(tmp_path, "g++", [os.path.join(HERE, "plan_driver.cpp"), os.path.join(csrc, "plan.cpp")],
                         ["-std=c++17", "-I", csrc])
    assert "0 failures" in out


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "gcc", [os.path.join(HERE, "oracle_driver.c"),
                                           os.path.join(ROOT, "oracle", "b2b_oracle.c")],
                         ["-std=c11", "-ffp-contract=off", "-lm", "-lpthread"])
    assert "checksum" in out
