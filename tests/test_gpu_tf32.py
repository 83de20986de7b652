"""GPU parity of the tf32 cascade (B2B_DTYPE_TF32: bf16 passes on the 32x32x16
instruction) against the oracle's tf32 cascade (operands rounded to tf32,
exact products, float32 sums).

Tolerances, from the arithmetic: three passes drop the product of the two
low parts, below 2^-14 of each product, and both sides round the
intermediates to tf32 (10 fraction bits), where a last-place difference of
the float32 sums can move a value across a rounding midpoint: a fraction p of
the intermediates, about (difference of the sums) / (tf32 spacing), then
differs by one tf32 unit, which leaves ~sqrt(p) 2^-11 of relative error in
D.  With differences of ~2^-18 (three passes) and ~2^-22 (four), that is
~5e-5 and ~1.5e-5 per intermediate; the bounds are relative Frobenius
<= 1e-3 for three passes (a one-pass bf16 emulation, operands rounded to 8
significant bits, misses it by ~3x) and <= 2e-4 for four, with per element
|d| <= 1e-2 (|ref| + 1).  Integer cases whose weights are exact
in bf16 make every dropped term zero and every partial sum an exact float32
integer: those compare bit for bit, and so does four-pass on integers whose
low parts multiply to nonzero values, where three passes cannot."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {3: 1e-3, 4: 2e-4}


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(batch, M, widths, seed=0x5EED0500):
    A = synth.tensor(seed, 0, (batch, M, widths[0]), "tf32", "normal", 1.0)
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), "tf32", "normal",
                       1.0 / math.sqrt(widths[s])) for s in range(len(widths) - 1)]
    return A, Bs


def _run(A, Bs, **kw):
    batch, M, K = A.shape
    widths = [K] + [b.shape[2] for b in Bs]
    Ad = torch.from_numpy(A).cuda()
    Bd = [torch.from_numpy(b).cuda() for b in Bs]
    D = torch.full((batch, M, widths[-1]), float("nan"), dtype=torch.float32, device="cuda")
    p = cf.Chain("tf32", batch, M, widths, **kw)
    info = p.info()
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    return D.cpu().numpy(), info


def _assert_exact_sums(A, Bs):
    """Every partial sum of every stage, in any order, is bounded by
    sum_k |x_k||b_k| over the tf32-rounded operands: below 2^24 it is an exact
    float32 integer."""
    for s in range(len(Bs)):
        X = A if s == 0 else oracle.cascade("tf32", A, Bs[:s])
        X = oracle.round_tf32(X).astype(np.float64)
        assert np.array_equal(X, np.round(X))
        assert (np.abs(X) @ np.abs(oracle.round_tf32(Bs[s])).astype(np.float64)).max() < 2 ** 24


def _close(got, ref, passes, what):
    g, r = got.astype(np.float64), ref.astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    fro = np.linalg.norm(g - r) / np.linalg.norm(r)
    assert fro <= TOL[passes], f"{what}: relative Frobenius error {fro:.3e}"
    bad = np.abs(g - r) > 1e-2 * (np.abs(r) + 1)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside 1e-2(|ref|+1)"
    return fro


CASES = [
    (2, 300, (128, 128, 128)),
    (1, 513, (64, 96, 32)),
    (3, 260, (128, 32, 128)),
    (1, 700, (128, 128, 128, 64)),      # three GEMMs
    (2, 333, (96, 64, 128, 32)),
    (2, 129, (64, 128)),                # one GEMM
]


@pytest.mark.parametrize("passes", [3, 4])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_tf32_parity(case, passes):
    batch, M, widths = CASES[case]
    _flush(f"tf32 x{passes} batch={batch} M={M} widths={widths}")
    A, Bs = _inputs(batch, M, widths)
    got, info = _run(A, Bs, tf32_exact=passes == 4)
    assert f"mfma=bf16x{passes}_32x32x16" in info and "path=fused" in info, info
    fro = _close(got, oracle.cascade("tf32", A, Bs), passes, f"tf32 x{passes} {widths}")
    print(f"relative Frobenius error {fro:.2e}", flush=True)


@pytest.mark.parametrize("passes", [3, 4])
def test_tf32_unfused(passes):
    widths = (128, 96, 128, 64, 32)
    _flush(f"tf32 unfused x{passes} widths={widths}")
    A, Bs = _inputs(2, 300, widths)
    got, info = _run(A, Bs, unfused=True, tf32_exact=passes == 4)
    assert "path=unfused" in info and "launches=4" in info, info
    _close(got, oracle.cascade("tf32", A, Bs), passes, f"tf32 unfused x{passes}")


@pytest.mark.parametrize("passes", [3, 4])
@pytest.mark.parametrize("widths", [(128, 128, 64), (64, 96, 128, 32), (128, 128, 128), (128, 128, 128, 64)])
def test_tf32_integers_exact(widths, passes):
    """A: integers up to 2047 (exact in tf32, low parts nonzero); weights
    ternary (exact in bf16, so no dropped term); the intermediates pass 2^11
    and are rounded to tf32; every partial sum is an integer below 2^24.
    The last two width sets run the instances with their widths compiled in."""
    _flush(f"tf32 exact x{passes} widths={widths}")
    rng = np.random.default_rng(41)
    A = rng.integers(-2047, 2048, (2, 300, widths[0])).astype(np.float32)
    Bs = [rng.integers(-1, 2, (2, widths[s], widths[s + 1])).astype(np.float32) for s in range(len(widths) - 1)]
    _assert_exact_sums(A, Bs)
    ref = oracle.cascade("tf32", A, Bs)
    got, info = _run(A, Bs, tf32_exact=passes == 4)
    compiled = widths in ((128, 128, 128), (128, 128, 128, 64))
    assert ("widths=compiled" in info) == compiled, info
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


def test_tf32_four_passes_exact_products():
    """Integers 257..700 in both operands: their low parts multiply to nonzero
    values, so only four passes give the exact tf32 products (every partial
    sum an integer below 2^24); three passes differ."""
    _flush("tf32 exact products")
    rng = np.random.default_rng(43)
    sign = lambda shape: rng.choice([-1.0, 1.0], shape)
    A = (rng.integers(257, 701, (2, 300, 32)) * sign((2, 300, 32))).astype(np.float32)
    B = (rng.integers(257, 701, (2, 32, 64)) * sign((2, 32, 64))).astype(np.float32)
    _assert_exact_sums(A, [B])
    ref = oracle.cascade("tf32", A, [B])
    got4, _ = _run(A, [B], tf32_exact=True)
    assert np.array_equal(got4, ref), f"{int((got4 != ref).sum())} elements differ"
    got3, _ = _run(A, [B])
    assert not np.array_equal(got3, ref)
    # the three-pass result misses exactly the low-part products, each below
    # 2^-14 |a b| (the sums stay exact integers)
    bound = 2.0 ** -14 * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64))
    assert np.all(np.abs(got3.astype(np.float64) - ref) <= bound)


def test_tf32_padded_and_broadcast():
    M, batch, widths = 300, 3, (64, 128, 96)
    _flush(f"tf32 strided widths={widths}")
    A, Bs = _inputs(batch, M, widths)
    Bs = [b.copy() for b in Bs]
    Bs[1][:] = Bs[1][0]                       # B_1 broadcast to every batch
    lda, ldd = widths[0] + 4, widths[-1] + 8
    ldb = [widths[1] + 4, widths[2] + 12]
    sA, sD = M * lda + 4, M * ldd + 12
    sB = [widths[0] * ldb[0] + 8, 0]

    def padded(x, b, rows, cols, ld, stride):
        buf = torch.full(((b - 1) * stride + rows * ld + 32,), float("nan"), dtype=torch.float32, device="cuda")
        buf.as_strided((b, rows, cols), (stride, ld, 1)).copy_(torch.from_numpy(x))
        return buf

    Ad = padded(A, batch, M, widths[0], lda, sA)
    Bd = [padded(Bs[0], batch, widths[0], widths[1], ldb[0], sB[0]),
          padded(Bs[1][:1], 1, widths[1], widths[2], ldb[1], 0)]
    Dd = torch.full(((batch - 1) * sD + M * ldd + 32,), float("nan"), dtype=torch.float32, device="cuda")
    p = cf.Chain("tf32", batch, M, widths, ld=[lda] + ldb + [ldd], batch_stride=[sA] + sB + [sD])
    p.run(Ad, *Bd, D=Dd)
    torch.cuda.synchronize()
    p.close()
    view = Dd.as_strided((batch, M, widths[-1]), (sD, ldd, 1))
    _close(view.cpu().numpy(), oracle.cascade("tf32", A, Bs), 3, "tf32 strided")
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, widths[-1]), (sD, ldd, 1)).fill_(False)
    assert torch.isnan(Dd[mask]).all().item(), "writes outside the output windows"
