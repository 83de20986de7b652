"""Seeded random sweep over the run-time-width kernels: widths drawn within
each family's granules and LDS bound, M from 1 to a few thousand (ragged),
batches 1-4, one to six GEMMs, both rearrangements, random type masks, tf32
with three and four passes, fp8 second GEMMs; every case against the
oracle."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close, check_fp8_stage, nan_output

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _widths(rng, nst, gran, maxd, bytes_per, budget=160 * 1024):
    while True:
        w = [int(rng.integers(1, maxd // gran + 1)) * gran for _ in range(nst + 1)]
        if sum(w[s] * w[s + 1] for s in range(nst)) * bytes_per <= budget:
            return w


def _case(i):
    rng = np.random.default_rng(0x5EED0900 + i)
    kind = ["16", "16", "typed", "tf32", "fp8"][i % 5]
    M = int(rng.choice([1, 31, 33, 255, 257]) if rng.random() < 0.3 else rng.integers(2, 3000))
    batch = int(rng.integers(1, 5))
    if kind == "16":
        nst = int(rng.integers(1, 5))
        dt = str(rng.choice(["f16", "bf16"]))
        mode = str(rng.choice(["relabel", "permlane"])) if nst > 1 else "relabel"
        maxd = 128 if (mode == "permlane" and nst > 3) else (256 if nst <= 3 else 128)
        return kind, [dt] * (nst + 1), _widths(rng, nst, 32, maxd, 2), M, batch, dict(mfma32=True, remap=mode)
    if kind == "typed":
        nst = int(rng.integers(2, 7))
        while True:
            types = [str(t) for t in rng.choice(["f16", "bf16"], nst + 1)]
            if len(set(types)) > 1:
                break
        return kind, types, _widths(rng, nst, 32, 256 if nst <= 3 else 128, 2), M, batch, {}
    if kind == "tf32":
        nst = int(rng.integers(1, 4))
        return kind, ["tf32"] * (nst + 1), _widths(rng, nst, 32, 128, 4), M, batch, dict(tf32_exact=bool(rng.random() < 0.5))
    t0, td = (str(t) for t in rng.choice(["f16", "bf16"], 2))
    while True:
        w = [int(rng.integers(1, 9)) * 32, int(rng.integers(1, 5)) * 64, int(rng.integers(1, 9)) * 32]
        if w[0] * w[1] * 2 + w[1] * w[2] <= 160 * 1024:
            break
    return kind, [t0, "fp8", td], w, M, batch, {}


@pytest.mark.parametrize("i", range(50))
def test_sweep_runtime_widths(i):
    kind, types, widths, M, batch, kw = _case(i)
    _flush(f"sweep {i}: {kind} types={types} widths={widths} M={M} batch={batch} {kw}")
    A = synth.tensor(0x5EED0A00 + i, 0, (batch, M, widths[0]), types[0], "normal")
    Bs = [synth.tensor(0x5EED0A00 + i, 1 + s, (batch, widths[s], widths[s + 1]), types[s], "normal",
                       1.0 / math.sqrt(widths[s])) for s in range(len(widths) - 1)]
    dtype = types[0] if len(set(types)) == 1 else list(types)
    p = cf.Chain(dtype, batch, M, widths, **kw)
    Ad = cf.to_device(A, types[0])
    Bd = [cf.to_device(b, types[s]) for s, b in enumerate(Bs)]
    if kind == "tf32":
        D = torch.full((batch, M, widths[-1]), float("nan"), dtype=torch.float32, device="cuda")
    else:
        D = nan_output(types[-1], batch, M, widths[-1])
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    got = cf.to_host(D)
    if kind == "tf32":
        ref = oracle.cascade("tf32", A, Bs).astype(np.float64)
        g = got.astype(np.float64)
        assert np.all(np.isfinite(g))
        tol = 2e-4 if kw["tf32_exact"] else 1e-3
        assert np.linalg.norm(g - ref) / np.linalg.norm(ref) <= tol
    elif kind == "fp8":
        def run(a, bs):
            Dx = nan_output(types[-1], batch, M, bs[1].shape[2])
            q = cf.Chain(dtype, batch, M, [widths[0], widths[1], bs[1].shape[2]])
            q.run(cf.to_device(a, types[0]), cf.to_device(bs[0], types[0]), cf.to_device(bs[1], "fp8"), D=Dx)
            torch.cuda.synchronize()
            q.close()
            return cf.to_host(Dx)
        check_fp8_stage(types, A, Bs[0], Bs[1], got, run, f"sweep {i}")
    else:
        assert_close(types[-1], got, oracle.cascade(dtype, A, Bs), f"sweep {i}")
