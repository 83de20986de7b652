"""GPU parity of the fp64 run-time-width kernels (v_mfma_f64_16x16x4): widths
that the fixed 64-wide kernel does not cover, one to five GEMMs, ragged M,
both ways of storing D (staged through LDS, and straight from registers when
the weights fill LDS), strided and broadcast layouts, the unfused per-GEMM
kernels of the same family, and exact ternary cases.  Tolerance: relative
Frobenius error <= 1e-12 against the fp64 oracle."""
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


def _inputs(batch, M, widths, dist="uniform", seed=0x5EED0300):
    A = synth.tensor(seed, 0, (batch, M, widths[0]), "f64", dist, 1.0)
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), "f64", dist,
                       1.0 if dist == "ternary" else 1.0 / math.sqrt(widths[s]))
          for s in range(len(widths) - 1)]
    return A, Bs


def _run(A, Bs, **kw):
    batch, M, K = A.shape
    widths = [K] + [b.shape[2] for b in Bs]
    Ad = cf.to_device(A, "f64")
    Bd = [cf.to_device(b, "f64") for b in Bs]
    D = nan_output("f64", batch, M, widths[-1])
    p = cf.Chain("f64", batch, M, widths, **kw)
    info = p.info()
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    return cf.to_host(D), info


CASES = [
    (2, 300, (96, 48, 112)),
    (1, 257, (8, 16, 16)),
    (3, 200, (128, 64, 128)),            # 128 KB of weights: D stored without staging
    (1, 500, (64, 96, 32, 80)),          # three GEMMs
    (2, 333, (64, 48, 64, 32, 64)),      # four
    (1, 400, (32, 64, 16, 64, 48, 32)),  # five
    (2, 129, (40, 16)),                  # one GEMM
    (2, 300, (96, 80, 96)),              # the instance bounded at 96 (one A tile ahead)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_f64_runtime_widths(case):
    batch, M, widths = CASES[case]
    _flush(f"gen64 batch={batch} M={M} widths={widths}")
    A, Bs = _inputs(batch, M, widths)
    got, info = _run(A, Bs)
    assert "mfma=f64_16x16x4" in info and "rows_per_wg=128" in info, info
    assert_close("f64", got, oracle.cascade("f64", A, Bs), f"gen64 {widths}")


@pytest.mark.parametrize("widths", [(96, 48, 112), (64, 48, 64, 32, 64), (96, 96, 48)])
def test_f64_ternary_exact(widths):
    _flush(f"gen64 ternary widths={widths}")
    A, Bs = _inputs(2, 300, widths, dist="ternary", seed=0x5EED0301)
    got, _ = _run(A, Bs)
    ref = oracle.cascade("f64", A, Bs)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("widths", [(96, 48, 112), (64, 96, 32, 80)])
def test_f64_unfused(widths):
    _flush(f"gen64 unfused widths={widths}")
    A, Bs = _inputs(2, 300, widths)
    got, info = _run(A, Bs, unfused=True)
    assert "path=unfused" in info and "mfma=f64_16x16x4" in info, info
    assert_close("f64", got, oracle.cascade("f64", A, Bs), f"gen64 unfused {widths}")


def test_f64_padded_and_broadcast():
    M, batch, widths = 300, 3, (48, 96, 32, 64)
    _flush(f"gen64 strided widths={widths}")
    A, Bs = _inputs(batch, M, widths)
    Bs = [b.copy() for b in Bs]
    Bs[1][:] = Bs[1][0]                       # B_1 broadcast to every batch
    nst = len(widths) - 1
    lda, ldd = widths[0] + 2, widths[-1] + 4
    ldb = [widths[s + 1] + 2 * (s + 1) for s in range(nst)]
    sA, sD = M * lda + 2, M * ldd + 6
    sB = [widths[s] * ldb[s] + 4 for s in range(nst)]
    sB[1] = 0

    def padded(x, b, rows, cols, ld, stride):
        buf = torch.full(((b - 1) * stride + rows * ld + 16,), float("nan"), dtype=torch.float64, device="cuda")
        buf.as_strided((b, rows, cols), (stride, ld, 1)).copy_(cf.to_device(x, "f64"))
        return buf

    Ad = padded(A, batch, M, widths[0], lda, sA)
    Bd = [padded(Bs[s] if s != 1 else Bs[s][:1], batch if s != 1 else 1, widths[s], widths[s + 1], ldb[s], sB[s])
          for s in range(nst)]
    Dd = torch.full(((batch - 1) * sD + M * ldd + 16,), float("nan"), dtype=torch.float64, device="cuda")
    p = cf.Chain("f64", batch, M, widths, ld=[lda] + ldb + [ldd], batch_stride=[sA] + sB + [sD])
    assert "mfma=f64_16x16x4" in p.info()
    p.run(Ad, *Bd, D=Dd)
    torch.cuda.synchronize()
    p.close()
    view = Dd.as_strided((batch, M, widths[-1]), (sD, ldd, 1))
    assert_close("f64", cf.to_host(view.contiguous()), oracle.cascade("f64", A, Bs), "gen64 strided")
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, widths[-1]), (sD, ldd, 1)).fill_(False)
    assert torch.isnan(Dd[mask]).all().item(), "writes outside the output windows"
