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
    """The cascade tolerance: relative Frobenius error, and for 16-bit types
    the per-element bound 2e-2 (|ref| + 1)."""
    g, r = values(dtype, got), values(dtype, ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output (unwritten or overflowed)"
    fro = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    assert fro <= TOL_FRO[dtype], f"{what}: relative Frobenius error {fro:.3e}"
    if dtype != "f64":
        bound = TOL_ELEM * (np.abs(r) + 1)
        bad = np.abs(g - r) > bound
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


def check_fp8_stage(types, A, B0, B1, got, run, what=""):
    """Checks a cascade {t0, fp8, tD} whose intermediate is rounded to E4M3.

    Where floating point decides a quantised code, the kernel and the oracle
    (summing in different orders) may round an intermediate that lies next to
    a midpoint to different neighbours.  So:
      1. the kernel's codes -- read back by running the same cascade with B1
         picking 64 columns at a time, which returns each fp8 intermediate
         exactly in tD -- equal
         the oracle's as values (so +0 and -0 agree), except where the oracle's fp32 sum lies within twice
         gamma_K sum_k |a_k b_k| (the dot-product error bound of either order,
         gamma_K = K 2^-24 / (1 - K 2^-24)) of a midpoint, and there the kernel
         took the other neighbour;
      2. D equals the oracle's cascade fed the kernel's codes, within the
         fp16/bf16 tolerance.
    run(A, [B0, B1]) runs the cascade and returns D's host encodings."""
    import oracle
    import synth
    t0, td = types[0], types[2]
    A, B0, B1 = (np.asarray(x) for x in (A, B0, B1))
    batch, M, K = A.shape
    N1 = B0.shape[2]
    # the kernel's fp8 intermediates, exactly: 64 columns at a time (B1 picking
    # columns c0 .. c0+63, so the weights stay within LDS at any width)
    X = np.empty((batch, M, N1))
    for c0 in range(0, N1, 64):
        sel = np.zeros((N1, 64))
        sel[c0 + np.arange(64), np.arange(64)] = 1.0
        X[:, :, c0:c0 + 64] = values(td, run(A, [B0, synth.to_dtype(np.broadcast_to(sel, (batch, N1, 64)), "fp8")]))
    codes_k = oracle.encode_fp8(X.astype(np.float32)).astype(np.int64)
    assert np.array_equal(oracle.decode_fp8(codes_k.astype(np.uint8)).astype(np.float64), X), f"{what}: not fp8"
    gamma = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    flips = 0
    for b in range(batch):
        x = oracle.gemm_acc(t0, A[b], B0[b]).astype(np.float64)
        win = 2 * gamma * (np.abs(values(t0, A[b])) @ np.abs(values(t0, B0[b])))
        codes_o = oracle.encode_fp8(x.astype(np.float32)).astype(np.int64)
        v = oracle.decode_fp8(codes_o.astype(np.uint8)).astype(np.float64)
        # compared as values: a negative intermediate that rounds to zero is
        # -0 in the oracle and +0 from the hardware conversion, equal numbers
        differ = X[b] != v
        if differ.any():
            w = X[b][differ]
            mid = (v[differ] + w) / 2
            # the kernel's value is the oracle's other neighbour, and x was within the window of the midpoint
            lo, hi = np.minimum(v[differ], w), np.maximum(v[differ], w)
            between = (x[differ] >= lo) & (x[differ] <= hi)
            assert between.all() and (np.abs(x[differ] - mid) <= win[differ]).all(), \
                f"{what}: {int(differ.sum())} intermediates rounded differently away from a tie"
            flips += int(differ.sum())
    X_td = synth.to_dtype(X, td)
    eye_td = synth.to_dtype(np.broadcast_to(np.eye(N1), (batch, N1, N1)), td)
    ref = oracle.cascade([td, "fp8", td], X_td, [eye_td, B1])
    assert_close(td, got, ref, what)
    return flips
