"""Host-side checks of bench.py: the workload arithmetic behind the roofline
object, and the one-GPU restriction (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

# Algorithmic FLOP = 2 batch M sum(d_s d_s+1); bytes = A + weights + D, each
# written out by hand from the workload shapes (no intermediate counted).
EXPECTED = {
    1: (2 * 1 * 128 * (64 * 64 + 64 * 64), 2 * (128 * 64 + 2 * 64 * 64 + 128 * 64)),
    2: (2 * 64 * 4096 * (128 * 128 * 2), 2 * 64 * (4096 * 128 + 2 * 128 * 128 + 4096 * 128)),
    3: (2 * 65536 * (256 * 256 * 2), 2 * (65536 * 256 + 2 * 256 * 256 + 65536 * 256)),
    4: (2 * 8 * 16384 * (64 * 64 * 2), 8 * 8 * (16384 * 64 + 2 * 64 * 64 + 16384 * 64)),
    5: (2 * 16 * 32768 * (128 * 128 * 2 + 128 * 64),
        2 * 16 * (32768 * 128 + 2 * 128 * 128 + 128 * 64 + 32768 * 64)),
}


@pytest.mark.parametrize("cfg", sorted(EXPECTED))
def test_workload_numbers(cfg):
    flop, byts = bench.workload_numbers(synth.WORKLOADS[cfg])
    assert (flop, byts) == EXPECTED[cfg]


def test_headline_flop_count():
    # 17.18 GFLOP for the 64 x 4096 x 128^3 fp16 workload
    assert abs(bench.workload_numbers(synth.WORKLOADS[2])[0] / 1e9 - 17.18) < 0.01


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_workload_numbers_per_stage_types():
    """An fp8 second GEMM counts its weights at one byte an element; tf32 at four."""
    c = dict(synth.WORKLOADS[2])
    flop, byts = bench.workload_numbers(c, ["f16", "fp8", "f16"])
    assert flop == EXPECTED[2][0]
    assert byts == 64 * (2 * 4096 * 128 + 2 * 128 * 128 + 1 * 128 * 128 + 2 * 4096 * 128)
    c["dtype"] = "tf32"
    assert bench.workload_numbers(c)[1] == 2 * EXPECTED[2][1]


@pytest.mark.parametrize("args", [["--types", "fp8,f16,f16"], ["--types", "f16,f16"], ["--types", "f16,f16,fp8"],
                                  ["--config", "4", "--types", "f64,f64,f64"], ["--tf32-exact"]])
def test_bad_type_options_refused(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r.stderr[-500:]
    assert r.stdout.strip() == ""
