"""Seeded sweep over the compiled shape families and many (M, batch) pairs --
tiny, one row either side of tile and wave boundaries, several workgroup
tiles, batches that straddle workgroup ranges -- against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import assert_close, run_plan

pytestmark = pytest.mark.gpu

FAMILIES = [
    ("f16", [64, 64, 64]),
    ("f16", [128, 128, 128]),
    ("f16", [128, 128, 128, 64]),
    ("bf16", [64, 64, 64]),
    ("bf16", [128, 128, 128]),
    ("bf16", [256, 256, 256]),
    ("f16", [256, 256, 256]),
    ("f64", [64, 64, 64]),
]
EDGE_M = [1, 2, 15, 16, 17, 31, 33, 63, 65, 127, 129, 255, 257, 511, 513]


def _pairs(seed, n=6):
    rng = np.random.default_rng(seed)
    ms = rng.choice(EDGE_M, size=n // 2, replace=False).tolist()
    ms += rng.integers(600, 2600, size=n - len(ms)).tolist()
    bs = rng.integers(1, 5, size=n).tolist()
    return list(zip(ms, bs))


def _inputs(dtype, dims, M, batch, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((batch, M, dims[0])) / np.sqrt(dims[0])
    Bs = [rng.standard_normal((batch, dims[s], dims[s + 1])) / np.sqrt(dims[s])
          for s in range(len(dims) - 1)]
    return synth.to_dtype(A, dtype), [synth.to_dtype(b, dtype) for b in Bs]


@pytest.mark.parametrize("fam", range(len(FAMILIES)))
def test_sweep(fam):
    dtype, dims = FAMILIES[fam]
    for i, (M, batch) in enumerate(_pairs(100 + fam)):
        print(f"\n[case] sweep {dtype} {dims} M={M} batch={batch}", flush=True)
        A, Bs = _inputs(dtype, dims, M, batch, seed=1000 * fam + i)
        got = run_plan(dtype, A, Bs)
        ref = oracle.cascade(dtype, A, Bs)
        assert_close(dtype, got, ref, f"{dtype} {dims} M={M} batch={batch}")


@pytest.mark.parametrize("fam", [0, 1, 2, 5, 7])
def test_sweep_unfused(fam):
    dtype, dims = FAMILIES[fam]
    for i, (M, batch) in enumerate(_pairs(200 + fam, n=3)):
        print(f"\n[case] sweep unfused {dtype} {dims} M={M} batch={batch}", flush=True)
        A, Bs = _inputs(dtype, dims, M, batch, seed=5000 + 1000 * fam + i)
        got = run_plan(dtype, A, Bs, unfused=True)
        ref = oracle.cascade(dtype, A, Bs)
        assert_close(dtype, got, ref, f"unfused {dtype} {dims} M={M} batch={batch}")
