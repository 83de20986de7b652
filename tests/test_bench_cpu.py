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


def test_roofline_binding_roof():
    # workload 5 is HBM-bound (212 FLOP/B against a ridge of 315), workload 4 fp64-MFMA-bound
    f5, b5 = bench.workload_numbers(synth.WORKLOADS[5])
    r = bench.roofline(f5, b5, 0.05, bench.PEAK["f16"])
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - b5 / 0.05e-3 / 1e9) < 1e-6 and abs(r["frac"] - r["achieved"] / 8000) < 1e-12
    f4, b4 = bench.workload_numbers(synth.WORKLOADS[4])
    r = bench.roofline(f4, b4, 0.04, bench.PEAK["f64"])
    assert r["bound"] == "mfma" and abs(r["achieved"] - f4 / 0.04e-3 / 1e12) < 1e-9


def test_repeats_cover_50_ms():
    assert bench.repeats_for(20.0, 5) == 5
    assert bench.repeats_for(4.2, 5) == 12        # 12 x 4.2 ms >= 50 ms
    assert bench.repeats_for(0.0, 5) > 5


def test_summarize_trace_keeps_the_last_launches(tmp_path):
    """Median, min and max over the last N launches of each kernel, in start order."""
    p = tmp_path / "kernel_trace.csv"
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    # kernel a: 10 warm-up launches of 100 ns, then 5 of 10..50 ns; kernel b: 2 launches
    t = 0
    for d in [100] * 10 + [10, 20, 30, 40, 50]:
        rows.append(f'"a<1, 2>",{t},{t + d}')
        t += 1000
    rows += ['"b",5,12', '"b",7,10']
    p.write_text("\n".join(rows) + "\n")
    out = {e["kernel"]: e for e in bench.summarize_trace(str(p), 5)}
    assert out["a<1, 2>"]["launches"] == 15 and out["a<1, 2>"]["timed"] == 5
    assert out["a<1, 2>"]["median_ns"] == 30 and out["a<1, 2>"]["min_ns"] == 10 and out["a<1, 2>"]["max_ns"] == 50
    assert out["b"]["median_ns"] == 5
