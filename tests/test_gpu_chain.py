"""GPU parity of cascades of any length (b2b_chain_create / b2b_chain_run):
four to six GEMMs on the run-time-width kernels in both rearrangements, one
GEMM, the two- and three-GEMM plans of the chain call against those of
b2b_gemm_create (bit for bit), the unfused chain against the fused one (bit
for bit, natural K order), exact ternary chains, and padded / broadcast
layouts.  Weights are drawn N(0, 1/rows) so every intermediate keeps unit
variance however long the chain."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close, nan_output

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(dtype, batch, M, widths, dist="normal", seed=0x5EED0200):
    A = synth.tensor(seed, 0, (batch, M, widths[0]), dtype, dist, 1.0)
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), dtype, dist,
                       1.0 / math.sqrt(widths[s]))
          for s in range(len(widths) - 1)]
    return A, Bs


def _run_chain(dtype, A, Bs, **kw):
    batch, M, K = A.shape
    widths = [K] + [b.shape[2] for b in Bs]
    Ad = cf.to_device(A, dtype)
    Bd = [cf.to_device(b, dtype) for b in Bs]
    D = nan_output(dtype, batch, M, widths[-1])
    p = cf.Chain(dtype, batch, M, widths, **kw)
    info = p.info()
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    return cf.to_host(D), info


CHAINS = [
    (2, 300, (128, 128, 128, 128, 64)),
    (1, 513, (64, 96, 128, 32, 128, 64, 128)),         # six GEMMs
    (3, 260, (96, 224, 64, 160, 32)),                  # widths above 128
    (1, 700, (256, 64, 256, 32, 96, 128)),             # five GEMMs
    (2, 300, (64, 96, 64, 128, 32, 64, 96, 64)),       # seven GEMMs
    (1, 513, (64, 64, 128, 64, 96, 32, 128, 64, 96)),  # eight GEMMs
]


# lane-half swaps are compiled for chains of up to six GEMMs up to 128 wide
LONG_CASES = [(c, dt, mode) for c in range(len(CHAINS)) for dt in ("f16", "bf16")
              for mode in ("relabel", "permlane")
              if mode == "relabel" or (max(CHAINS[c][2]) <= 128 and len(CHAINS[c][2]) <= 7)]


@pytest.mark.parametrize("case,dtype,mode", LONG_CASES)
def test_long_chains(case, dtype, mode):
    batch, M, widths = CHAINS[case]
    _flush(f"chain {dtype} {mode} batch={batch} M={M} widths={widths}")
    A, Bs = _inputs(dtype, batch, M, widths)
    got, info = _run_chain(dtype, A, Bs, remap=mode)
    assert "mfma=32x32x16" in info and f"remap={mode}" in info, info
    assert_close(dtype, got, oracle.cascade(dtype, A, Bs), f"chain {widths} {mode}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_long_chain_ternary_exact(dtype):
    widths = (64, 96, 128, 32, 64)
    _flush(f"chain ternary {dtype} widths={widths}")
    A, Bs = _inputs(dtype, 2, 300, widths, dist="ternary", seed=0x5EED0201)
    got, _ = _run_chain(dtype, A, Bs)
    ref = oracle.cascade(dtype, A, Bs)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_unfused_chain_matches_fused_bitwise(dtype):
    widths = (128, 96, 128, 64, 32)
    _flush(f"chain unfused vs fused {dtype} widths={widths}")
    A, Bs = _inputs(dtype, 2, 300, widths)
    fused, _ = _run_chain(dtype, A, Bs, remap="permlane")
    unf, info = _run_chain(dtype, A, Bs, unfused=True, mfma32=True)
    assert "path=unfused" in info and "launches=4" in info, info
    assert np.array_equal(fused, unf), f"{int((fused != unf).sum())} elements differ"


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_short_chains_match_gemm_api(cfg):
    """Up to three GEMMs the chain call plans and runs exactly what
    b2b_gemm_create does (fp64 included)."""
    c = synth.WORKLOADS[cfg]
    dt, dims = c["dtype"], c["dims"]
    M, batch = min(c["M"], 300), min(c["batch"], 2)
    _flush(f"chain vs gemm api cfg{cfg}")
    A, Bs = synth.make_inputs(cfg, M=M, batch=batch)
    got, info = _run_chain(dt, A, Bs)
    Ad = cf.to_device(A, dt)
    Bd = [cf.to_device(b, dt) for b in Bs]
    D = nan_output(dt, batch, M, dims[-1])
    p = cf.Plan(dt, batch, M, *dims[:3], dims[3] if len(dims) > 3 else 0)
    assert p.info().split(" grid=")[0] == info.split(" grid=")[0]
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    assert np.array_equal(got, cf.to_host(D))


@pytest.mark.parametrize("widths,dtype", [((128, 128), "f16"), ((96, 160), "bf16"), ((64, 64), "f64")])
def test_single_gemm(widths, dtype):
    _flush(f"chain of one {dtype} {widths}")
    A, Bs = _inputs(dtype, 2, 300, widths)
    got, _ = _run_chain(dtype, A, Bs)
    assert_close(dtype, got, oracle.cascade(dtype, A, Bs), f"one GEMM {widths}")


def test_chain_padded_and_broadcast():
    dt, M, batch, widths = "f16", 300, 3, (96, 128, 64, 128, 32)
    _flush(f"chain strided widths={widths}")
    A, Bs = _inputs(dt, batch, M, widths)
    Bs = [b.copy() for b in Bs]
    Bs[2][:] = Bs[2][0]                       # B_2 broadcast to every batch
    nst = len(widths) - 1
    lda, ldd = widths[0] + 8, widths[-1] + 16
    ldb = [widths[s + 1] + 8 * (s % 2 + 1) for s in range(nst)]
    sA, sD = M * lda + 8, M * ldd + 24
    sB = [widths[s] * ldb[s] + 16 for s in range(nst)]
    sB[2] = 0

    def padded(x, b, rows, cols, ld, stride):
        buf = torch.full(((b - 1) * stride + rows * ld + 64,), float("nan"), dtype=torch.float16, device="cuda")
        buf.as_strided((b, rows, cols), (stride, ld, 1)).copy_(cf.to_device(x, dt))
        return buf

    Ad = padded(A, batch, M, widths[0], lda, sA)
    Bd = [padded(Bs[s] if s != 2 else Bs[s][:1], batch if s != 2 else 1, widths[s], widths[s + 1], ldb[s], sB[s])
          for s in range(nst)]
    Dd = torch.full(((batch - 1) * sD + M * ldd + 64,), float("nan"), dtype=torch.float16, device="cuda")
    p = cf.Chain(dt, batch, M, widths, ld=[lda] + ldb + [ldd], batch_stride=[sA] + sB + [sD])
    p.run(Ad, *Bd, D=Dd)
    torch.cuda.synchronize()
    p.close()
    view = Dd.as_strided((batch, M, widths[-1]), (sD, ldd, 1))
    assert_close(dt, cf.to_host(view.contiguous()), oracle.cascade(dt, A, Bs), "chain strided")
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, widths[-1]), (sD, ldd, 1)).fill_(False)
    assert torch.isnan(Dd[mask]).all().item(), "writes outside the output windows"
