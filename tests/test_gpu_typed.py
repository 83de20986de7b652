"""GPU parity of cascades with a 16-bit type per stage (b2b_chain_create_typed):
GEMM s computes in its own type, its result is rounded into the next GEMM's
type, D into the last one.  Fused two- and three-GEMM cascades on the 32x32x16
kernels, unfused cascades of any length, against the oracle's typed cascade
within the fp16/bf16 tolerances; integer cases whose intermediates exceed the
exact integer range of their type (256 in bf16, 2048 in fp16) compare bit for
bit, so a rounding into the wrong type fails them."""
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


def _normal_inputs(types, batch, M, widths, seed=0x5EED0400):
    A = synth.tensor(seed, 0, (batch, M, widths[0]), types[0], "normal", 1.0)
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), types[s], "normal",
                       1.0 / math.sqrt(widths[s])) for s in range(len(widths) - 1)]
    return A, Bs


def _run(types, A, Bs, **kw):
    batch, M, K = A.shape
    widths = [K] + [b.shape[2] for b in Bs]
    Ad = cf.to_device(A, types[0])
    Bd = [cf.to_device(b, types[s]) for s, b in enumerate(Bs)]
    D = nan_output(types[-1], batch, M, widths[-1])
    p = cf.Chain(list(types), batch, M, widths, **kw)
    info = p.info()
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    return cf.to_host(D), info


FUSED = [
    (("f16", "bf16", "f16"), 2, 300, (128, 128, 128)),
    (("bf16", "f16", "bf16"), 1, 513, (256, 256, 64)),
    (("f16", "f16", "bf16"), 3, 260, (96, 160, 32)),
    (("bf16", "bf16", "f16"), 1, 700, (64, 224, 128)),
    (("f16", "bf16", "f16", "bf16"), 2, 333, (128, 96, 128, 64)),
    (("bf16", "f16", "f16", "f16"), 1, 257, (64, 128, 32, 128)),
    (("f16", "f16", "f16", "bf16"), 2, 100, (128, 128, 128, 64)),
    # mixtures read at run time: three to five GEMMs past 128 wide, four to seven GEMMs
    (("f16", "bf16", "f16", "bf16"), 2, 300, (256, 64, 256, 64)),
    (("f16", "bf16", "bf16", "f16", "f16"), 2, 333, (128, 128, 128, 128, 64)),
    (("bf16", "f16", "bf16", "f16", "bf16", "f16"), 1, 513, (64, 96, 128, 32, 128, 64)),
    (("bf16", "f16", "bf16", "f16", "bf16", "f16", "bf16"), 2, 257, (64, 96, 128, 32, 128, 64, 128)),
    (("f16", "f16", "bf16", "f16", "bf16", "bf16", "f16", "bf16"), 2, 300, (64, 96, 64, 128, 32, 64, 96, 64)),
    # four and five GEMMs past 128 wide
    (("f16", "bf16", "f16", "bf16", "f16"), 2, 300, (256, 128, 128, 128, 64)),
    (("bf16", "f16", "bf16", "f16", "bf16", "f16"), 3, 257, (256, 64, 192, 64, 128, 64)),
    (("bf16", "f16", "f16", "bf16", "bf16", "f16", "bf16", "f16", "bf16"), 1, 513, (64, 64, 128, 64, 96, 32, 128, 64, 96)),
]


@pytest.mark.parametrize("case", range(len(FUSED)))
def test_typed_fused(case):
    types, batch, M, widths = FUSED[case]
    _flush(f"typed fused {types} batch={batch} M={M} widths={widths}")
    A, Bs = _normal_inputs(types, batch, M, widths)
    got, info = _run(types, A, Bs)
    assert "path=fused" in info and "dtype=" + "/".join(types) in info and "mfma=32x32x16" in info, info
    assert_close(types[-1], got, oracle.cascade(list(types), A, Bs), f"typed {types} {widths}")


@pytest.mark.parametrize("types,widths", [(("f16", "bf16", "bf16", "f16", "f16"), (128, 128, 96, 128, 64)),
                                          (("bf16", "f16", "bf16"), (128, 64, 128))])
def test_typed_unfused(types, widths):
    _flush(f"typed unfused {types} widths={widths}")
    A, Bs = _normal_inputs(types, 2, 300, widths)
    got, info = _run(types, A, Bs, unfused=True)
    assert "path=unfused" in info and f"launches={len(widths) - 1}" in info, info
    assert_close(types[-1], got, oracle.cascade(list(types), A, Bs), f"typed unfused {types}")


def _integer_inputs(types, widths, lims, batch=2, M=300, seed=23):
    """A and B_0 .. B_{n-2} non-negative integers up to lims[s] (so the
    intermediates grow past the exact range), the last B ternary (so D stays
    in range); every partial sum is an integer below 2^24, exact in fp32."""
    rng = np.random.default_rng(seed)
    A = synth.to_dtype(rng.integers(0, lims[0] + 1, (batch, M, widths[0])), types[0])
    Bs = []
    n = len(widths) - 1
    for s in range(n):
        shape = (batch, widths[s], widths[s + 1])
        vals = rng.integers(-1, 2, shape) if s == n - 1 else rng.integers(0, lims[s + 1] + 1, shape)
        Bs.append(synth.to_dtype(vals, types[s]))
    return A, Bs


@pytest.mark.parametrize("types,widths,lims,kw", [
    (("f16", "bf16", "f16"), (128, 128, 64), (3, 3), {}),
    (("bf16", "f16", "bf16"), (128, 128, 64), (7, 7), {}),
    (("f16", "bf16", "f16", "bf16"), (64, 64, 32, 64), (3, 3, 1), {}),
    (("f16", "bf16", "f16"), (128, 128, 64), (3, 3), {"unfused": True}),
    (("f16", "bf16", "f16", "bf16", "bf16"), (64, 32, 32, 32, 64), (3, 2, 1, 1), {}),  # run-time types
])
def test_typed_integer_exact(types, widths, lims, kw):
    _flush(f"typed exact {types} widths={widths} {kw}")
    A, Bs = _integer_inputs(types, widths, lims)
    ref = oracle.cascade(list(types), A, Bs)
    # the types matter: the same inputs read in one type give another result
    other = oracle.cascade(types[0], A, [synth.to_dtype(oracle.decode(types[s], b), types[0])
                                         for s, b in enumerate(Bs)])
    assert not np.array_equal(oracle.decode(types[-1], ref), oracle.decode(types[0], other))
    got, _ = _run(types, A, Bs, **kw)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


@pytest.mark.parametrize("types,widths", [
    (("bf16", "f16", "f16", "bf16"), (64, 96, 128, 32)),
    (("f16", "bf16", "bf16", "f16", "bf16"), (64, 96, 128, 32, 64)),     # run-time types
])
def test_typed_padded_and_broadcast(types, widths):
    M, batch = 300, 3
    _flush(f"typed strided {types} widths={widths}")
    A, Bs = _normal_inputs(types, batch, M, widths)
    Bs = [b.copy() for b in Bs]
    Bs[1][:] = Bs[1][0]                       # B_1 broadcast to every batch
    nst = len(widths) - 1
    lda, ldd = widths[0] + 8, widths[-1] + 16
    ldb = [widths[s + 1] + 8 * (s + 1) for s in range(nst)]
    sA, sD = M * lda + 8, M * ldd + 24
    sB = [widths[s] * ldb[s] + 16 for s in range(nst)]
    sB[1] = 0

    def padded(x, b, rows, cols, ld, stride, t):
        dt = cf.TORCH_DTYPES[cf.DTYPES[t]]
        buf = torch.full(((b - 1) * stride + rows * ld + 64,), float("nan"), dtype=dt, device="cuda")
        buf.as_strided((b, rows, cols), (stride, ld, 1)).copy_(cf.to_device(x, t))
        return buf

    Ad = padded(A, batch, M, widths[0], lda, sA, types[0])
    Bd = [padded(Bs[s] if s != 1 else Bs[s][:1], batch if s != 1 else 1, widths[s], widths[s + 1], ldb[s], sB[s],
                 types[s]) for s in range(nst)]
    Dd = torch.full(((batch - 1) * sD + M * ldd + 64,), float("nan"), dtype=cf.TORCH_DTYPES[cf.DTYPES[types[-1]]],
                    device="cuda")
    p = cf.Chain(list(types), batch, M, list(widths), ld=[lda] + ldb + [ldd], batch_stride=[sA] + sB + [sD])
    assert "path=fused" in p.info(), p.info()
    p.run(Ad, *Bd, D=Dd)
    torch.cuda.synchronize()
    p.close()
    view = Dd.as_strided((batch, M, widths[-1]), (sD, ldd, 1))
    assert_close(types[-1], cf.to_host(view.contiguous()), oracle.cascade(list(types), A, Bs), "typed strided")
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, widths[-1]), (sD, ldd, 1)).fill_(False)
    assert torch.isnan(Dd[mask]).all().item(), "writes outside the output windows"
