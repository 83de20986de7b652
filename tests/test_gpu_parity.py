"""GPU parity: the HIP path through the C ABI against the CPU oracle."""
import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from oracle import remap as R
from gpu_common import assert_close, run_plan

pytestmark = pytest.mark.gpu

MODES_T = ["relabel", "permlane", "bpermute", "lds"]
MODES_N = ["bpermute", "lds"]


def _flush(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# The device rearrangement executors against the oracle's relation, bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", ["f16_16x16x32", "bf16_16x16x32", "f64_16x16x4"])
@pytest.mark.parametrize("mode,orient", [(m, "T") for m in MODES_T] + [(m, "N") for m in MODES_N])
def test_remap_probe_bit_exact(shape, mode, orient):
    _flush(f"probe {shape} {mode} {orient}")
    src, dst, meta = R.cascade_layouts(shape, orient)
    rel = np.array(R.relation(src, dst))
    E = meta["elems"]
    n = 64 * E
    if shape.startswith("f64"):
        payload = torch.arange(n, dtype=torch.int64, device="cuda") * 0x10001 + 0x3FF0000000000000
        inp = payload.view(torch.float64)
    else:
        inp = (torch.arange(n, dtype=torch.int32, device="cuda") * 97 + 5).to(torch.int16)
    out = cf.remap_probe(shape, mode, inp, orient_n=(orient == "N"))
    torch.cuda.synchronize()
    i = inp.view(torch.int64 if shape.startswith("f64") else torch.int16).cpu().numpy()
    o = out.view(torch.int64 if shape.startswith("f64") else torch.int16).cpu().numpy()
    if mode == "relabel":
        # RELABEL moves nothing: the next GEMM reads the accumulator registers as they are
        assert np.array_equal(o, i)
    else:
        assert np.array_equal(o, i[rel]), f"{int((o != i[rel]).sum())} of {n} elements misplaced"


# ---------------------------------------------------------------------------
# Whole cascade at reduced sizes: several tiles and a ragged tail of M
# ---------------------------------------------------------------------------
SMALL = {1: dict(M=128, batch=1), 2: dict(M=1000, batch=3), 4: dict(M=777, batch=2),
         5: dict(M=600, batch=2)}


def _cases():
    for cfg in (1, 2, 4, 5):
        for m in MODES_T:
            yield cfg, m, False
        for m in MODES_N:
            yield cfg, m, True


@pytest.mark.parametrize("cfg,mode,orient_n", list(_cases()))
def test_cascade_parity_small(cfg, mode, orient_n):
    c = synth.WORKLOADS[cfg]
    _flush(f"cascade cfg{cfg} {mode} orientN={orient_n} {SMALL[cfg]}")
    A, Bs = synth.make_inputs(cfg, **SMALL[cfg])
    got = run_plan(c["dtype"], A, Bs, remap=mode, orient_n=orient_n)
    ref = oracle.cascade(c["dtype"], A, Bs)
    assert_close(c["dtype"], got, ref, f"cfg{cfg} {mode}")


@pytest.mark.parametrize("cfg,mode,orient_n", list(_cases()))
def test_cascade_ternary_bit_exact(cfg, mode, orient_n):
    """Small-integer inputs: every partial sum is exact in the accumulator, so
    any summation order gives the oracle's result bit for bit."""
    c = synth.WORKLOADS[cfg]
    _flush(f"ternary cfg{cfg} {mode} orientN={orient_n}")
    A, Bs = synth.make_inputs(cfg, dist="ternary", **SMALL[cfg])
    got = run_plan(c["dtype"], A, Bs, remap=mode, orient_n=orient_n)
    ref = oracle.cascade(c["dtype"], A, Bs)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_unfused_path_parity(cfg):
    c = synth.WORKLOADS[cfg]
    _flush(f"unfused cfg{cfg}")
    A, Bs = synth.make_inputs(cfg, **SMALL[cfg])
    got = run_plan(c["dtype"], A, Bs, unfused=True)
    ref = oracle.cascade(c["dtype"], A, Bs)
    assert_close(c["dtype"], got, ref, f"unfused cfg{cfg}")


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
@pytest.mark.parametrize("mode", ["permlane", "bpermute", "lds"])
def test_fused_equals_unfused_bitwise(cfg, mode):
    """With the natural K order the fused kernel issues the same MFMA chain as
    the two-kernel path, whose intermediate goes through HBM already rounded:
    the results must agree bit for bit."""
    c = synth.WORKLOADS[cfg]
    _flush(f"fused==unfused cfg{cfg} {mode}")
    A, Bs = synth.make_inputs(cfg, **SMALL[cfg])
    f = run_plan(c["dtype"], A, Bs, remap=mode)
    u = run_plan(c["dtype"], A, Bs, unfused=True)
    assert np.array_equal(f, u)


# ---------------------------------------------------------------------------
# Full workload sizes, in the launch configuration the benchmark times:
# every row written (D pre-filled with NaN), sampled rows against the oracle
# ---------------------------------------------------------------------------
def _sample_rows(batch, M, n=384, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.integers(0, batch * M, n).tolist())
    for b in range(batch):            # first and last rows of every batch
        rows.update([b * M, b * M + M - 1])
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_sampled(cfg):
    c = synth.WORKLOADS[cfg]
    dt, dims = c["dtype"], c["dims"]
    _flush(f"full size cfg{cfg}: batch {c['batch']} M {c['M']} dims {dims}")
    A, Bs = synth.make_inputs(cfg)
    Ad = cf.to_device(A, dt)
    Bd = [cf.to_device(b, dt) for b in Bs]
    D = torch.full((c["batch"], c["M"], dims[-1]), float("nan"), dtype=Ad.dtype, device="cuda")
    p = cf.Plan(dt, c["batch"], c["M"], *dims[:3], dims[3] if len(dims) > 3 else 0)
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    assert not torch.isnan(D).any().item(), "unwritten output elements"
    rows = _sample_rows(c["batch"], c["M"])
    got = cf.to_host(D).reshape(-1, dims[-1])[rows]
    ref = oracle.cascade(dt, A, Bs, rows=rows)
    assert_close(dt, got, ref, f"cfg{cfg} full size")
    p.close()


# ---------------------------------------------------------------------------
# Rounding of the intermediate and of D: round to nearest, ties to even
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rounding_is_nearest_even(dtype):
    """C0 = x + f*ulp(x) with f in {1/4, 1/2, 3/4} (exact in float32), B1 = I:
    then D = rnd(C0) exactly.  Round-to-nearest-even gives the oracle's bits;
    truncation (RTZ) or ties-away differ on the quarter and half cases."""
    M, K, N = 64, 32, 32
    sig = 11 if dtype == "f16" else 8
    rng = np.random.default_rng(9)
    A = np.zeros((M, K)); B0 = np.zeros((K, N))
    # x = (1 + j/2^(sig-1)) * 2^e on the diagonal-like first column, fraction via the second
    e = rng.integers(-3, 4, (M, 1))
    A[:, 0] = 2.0 ** e[:, 0]
    frac = rng.choice([0.25, 0.5, 0.75], size=M)
    A[:, 1] = frac * 2.0 ** (e[:, 0] - (sig - 1))
    B0[0, :] = 1.0 + rng.integers(0, 2 ** (sig - 1), N) / 2.0 ** (sig - 1)
    B0[1, :] = 1.0
    # the supported widths: embed the 32-wide problem in the 64-wide kernel with zero padding
    Ap = np.zeros((1, M, 64), np.float64); Ap[0, :, :K] = A
    B0p = np.zeros((64, 64)); B0p[:K, :N] = B0
    B1p = np.eye(64)
    Ae = synth.to_dtype(Ap, dtype)
    Be = [synth.to_dtype(B0p, dtype)[None], synth.to_dtype(B1p, dtype)[None]]
    ref = oracle.cascade(dtype, Ae, Be)
    assert np.array_equal(oracle.decode(dtype, Ae).astype(np.float64), Ap)    # exact inputs
    for mode in (MODES_T if dtype == "f16" else ["relabel", "permlane"]):
        got = run_plan(dtype, Ae, Be, remap=mode)
        assert np.array_equal(got, ref), mode
    vals = oracle.decode(dtype, ref[0, :, :N]).astype(np.float64)
    exact = (A[:, :1] * B0[:1, :] + A[:, 1:2] * B0[1:2, :])
    assert np.any(vals != exact)          # rounding really happened


# ---------------------------------------------------------------------------
# Weights larger than LDS (two 256x256 matrices): column-split kernel whose
# rearrangement goes through LDS across the workgroup's waves
# ---------------------------------------------------------------------------
# (4000, 3): 375 tiles over 256 workgroups, so some workgroups run two
# tiles that straddle a batch boundary (two weight segments)
@pytest.mark.parametrize("M,batch", [(1000, 1), (777, 2), (32, 1), (1, 1), (4000, 3)])
def test_wide_cascade_parity(M, batch):
    _flush(f"wide cascade bf16 256^3 M={M} batch={batch}")
    A, Bs = synth.make_inputs(3, M=M, batch=batch)
    got = run_plan("bf16", A, Bs)
    ref = oracle.cascade("bf16", A, Bs)
    assert_close("bf16", got, ref, f"bf16 256^3 M={M}")


def test_wide_cascade_ternary_bit_exact():
    _flush("wide cascade ternary")
    A, Bs = synth.make_inputs(3, M=500, batch=2, dist="ternary")
    assert np.array_equal(run_plan("bf16", A, Bs), oracle.cascade("bf16", A, Bs))


def test_wide_cascade_f16_parity():
    """The same column-split kernel instantiated for fp16."""
    A, Bs = synth.make_inputs(dict(synth.WORKLOADS[3], dtype="f16"), M=600, batch=1)
    f = run_plan("f16", A, Bs)
    ref = oracle.cascade("f16", A, Bs)
    assert_close("f16", f, ref, "f16 256^3")
