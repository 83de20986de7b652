"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU): the
planner that derives the relations and exchange rounds (plan.cpp) and the C
oracle, each built with gcc/g++ and both sanitizers into a small driver that
exercises every shape and orientation, random relations, and cascades of
every type at odd sizes on one and several threads.  Any sanitizer report
ends the driver with a nonzero status.  The planner is built with its
B2B_DEBUG bounds and invariant checks on; one run plants an out-of-range
element index and expects the check to abort."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build(tmp_path, compiler, srcs, extra):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / "driver")
    r = subprocess.run([compiler] + SAN + srcs + extra + ["-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    return exe, env


def _build_and_run(tmp_path, compiler, srcs, extra):
    exe, env = _build(tmp_path, compiler, srcs, extra)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-4000:]
    return run.stdout


CSRC = os.path.join(ROOT, "chip_fusion_amd", "csrc")
PLAN_SRCS = [os.path.join(HERE, "plan_driver.cpp"), os.path.join(CSRC, "plan.cpp")]
PLAN_FLAGS = ["-std=c++17", "-DB2B_DEBUG", "-I", CSRC]


def test_planner_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "g++", PLAN_SRCS, PLAN_FLAGS)
    assert "0 failures" in out


def test_planner_debug_check_fires(tmp_path):
    exe, env = _build(tmp_path, "g++", PLAN_SRCS, PLAN_FLAGS)
    run = subprocess.run([exe, "--out-of-range"], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode != 0 and "no check fired" not in run.stdout
    assert "B2B_DEBUG check failed: e >= 0 && e < sh.a_elems" in run.stderr, run.stderr[-2000:]


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "gcc", [os.path.join(HERE, "oracle_driver.c"),
                                           os.path.join(ROOT, "oracle", "b2b_oracle.c")],
                         ["-std=c11", "-ffp-contract=off", "-lm", "-lpthread"])
    assert "checksum" in out
