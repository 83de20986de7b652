"""Helpers shared by the GPU parity tests (comparison rules, device copies)."""
import numpy as np
import torch

import chip_fusion_amd as cf
import oracle

# Tolerances (fp16/bf16: relative Frobenius <= 5e-3 and per element
# |d| <= 2e-2 (|ref| + 1); fp64: relative Frobenius <= 1e-12).
TOL_FRO = {"f16": 5e-3, "bf16": 5e-3, "f64": 1e-12}
TOL_ELEM = 2e-2


def values(dtype, x):
    return oracle.decode(dtype, x).astype(np.float64)


def assert_close(dtype, got, ref, what=""):
    g, r = values(dtype, got), values(dtype, ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output (unwritten or overflowed)"
    fro = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    assert fro <= TOL_FRO[dtype], f"{what}: relative Frobenius error {fro:.3e}"
    if dtype != "f64":
        bad = np.abs(g - r) > TOL_ELEM * (np.abs(r) + 1)
        assert not bad.any(), f"{what}: {int(bad.sum())} elements outside 2e-2(|ref|+1)"
    return fro


def device_inputs(dtype, A, Bs):
    return cf.to_device(A, dtype), [cf.to_device(b, dtype) for b in Bs]


def nan_output(dtype, batch, M, N):
    tdt = cf.TORCH_DTYPES[cf.DTYPES[dtype]]
    return torch.full((batch, M, N), float("nan"), dtype=tdt, device="cuda")


def run_plan(dtype, A, Bs, remap="auto", orient_n=False, unfused=False):
    """Runs the cascade on the GPU through the C ABI; returns host encodings."""
    batch, M, K = A.shape
    dims = [K] + [b.shape[2] for b in Bs]
    Ad, Bd = device_inputs(dtype, A, Bs)
    D = nan_output(dtype, batch, M, dims[-1])
    p = cf.Plan(dtype, batch, M, *dims, remap=remap, orient_n=orient_n, unfused=unfused)
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    out = cf.to_host(D)
    p.close()
    return out
