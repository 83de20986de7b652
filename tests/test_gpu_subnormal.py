"""Subnormal numbers through the whole GPU path, bit for bit against the oracle
(which follows IEEE 754 gradual underflow).

Inputs are small integers times the smallest subnormal of the type, weights
small integers, so every product and partial sum is exact in the accumulator
(fp32 holds them; fp64 holds the fp64 ones) and the only rounding is the
conversion of the results into the type: B1 = I/2 makes half of the results
fall on a midpoint of the subnormal grid, so round-half-even is exercised in
the subnormal range too.  A flush-to-zero anywhere (inputs, accumulator,
conversion) changes the result."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import run_plan

pytestmark = pytest.mark.gpu

# smallest subnormal of each type, and the largest integer multiple used
TINY = {"f16": 2.0 ** -24, "bf16": 2.0 ** -133, "f64": 2.0 ** -1074}
SPAN = {"f16": 8, "bf16": 8, "f64": 8}


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f64"])
def test_subnormals_bit_exact(dtype):
    print(f"\n[case] subnormals {dtype}", flush=True)
    rng = np.random.default_rng(11)
    M, K, N1, N2 = 200, 64, 64, 64
    A = rng.integers(-SPAN[dtype], SPAN[dtype] + 1, (1, M, K)) * TINY[dtype]
    B0 = rng.integers(-3, 4, (1, K, N1)).astype(np.float64)
    B1 = 0.5 * np.eye(N1, N2)[None]
    Ae = synth.to_dtype(A, dtype)
    Be = [synth.to_dtype(B0, dtype), synth.to_dtype(B1, dtype)]
    # the encodings really are the intended values (subnormal inputs)
    assert np.array_equal(oracle.decode(dtype, Ae).astype(np.float64), A)
    ref = oracle.cascade(dtype, Ae, Be)
    vals = oracle.decode(dtype, ref).astype(np.float64)
    assert np.count_nonzero(vals) > vals.size // 2          # not flushed in the oracle either
    c0 = np.einsum("bmk,bkn->bmn", A, B0)                   # exact (small integers x tiny)
    assert np.any((np.abs(c0 / TINY[dtype]) % 2) == 1)      # odd multiples: midpoints after x 1/2
    got = run_plan(dtype, Ae, Be)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of {got.size} results differ"
