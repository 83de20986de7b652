"""GPU parity of the run-time-width kernels on the 32x32x16 instruction:
widths that no fixed-width kernel covers, the configurations' widths forced
onto this path, both rearrangements (relabelled K order, lane-half swaps),
two and three GEMMs, ragged M, padded and broadcast layouts, and the unfused
per-GEMM kernels of the same family.  Gaussian inputs are checked against the
oracle within the tolerance; ternary inputs, whose sums are exact in fp32,
bit for bit."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close, device_inputs, nan_output

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(dtype, batch, M, dims, dist="normal", seed=0x5EED0100):
    scale = 1.0 / math.sqrt(max(dims))
    cfg = dict(dtype=dtype, batch=batch, M=M, dims=list(dims), dist=dist, scale=scale, seed=seed)
    return synth.make_inputs(cfg)


def _run(dtype, A, Bs, **kw):
    batch, M, K = A.shape
    dims = [K] + [b.shape[2] for b in Bs]
    Ad, Bd = device_inputs(dtype, A, Bs)
    D = nan_output(dtype, batch, M, dims[-1])
    p = cf.Plan(dtype, batch, M, *dims, **kw)
    info = p.info()
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    return cf.to_host(D), info


# (batch, M, widths): odd multiples of 32, K of 16, ragged M, several tiles
SHAPES = [
    (2, 300, (96, 160, 64)),
    (1, 257, (32, 32, 32)),
    (3, 520, (32, 224, 96)),
    (1, 700, (256, 128, 256)),          # 128 KB of weights
    (2, 333, (64, 192, 96, 32)),        # three GEMMs
    (1, 513, (160, 96, 256, 64)),
    (1, 400, (224, 160, 224)),          # 140 KB of weights: D stored without staging
]


@pytest.mark.parametrize("mode", ["relabel", "permlane"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_runtime_widths(case, dtype, mode):
    batch, M, dims = SHAPES[case]
    _flush(f"gen {dtype} {mode} batch={batch} M={M} dims={dims}")
    A, Bs = _inputs(dtype, batch, M, dims)
    got, info = _run(dtype, A, Bs, remap=mode)
    assert "mfma=32x32x16" in info and f"remap={mode}" in info, info
    assert_close(dtype, got, oracle.cascade(dtype, A, Bs), f"gen {dims} {mode}")


@pytest.mark.parametrize("mode", ["relabel", "permlane"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("dims", [(96, 160, 64), (64, 192, 96, 32), (256, 128, 256)])
def test_runtime_widths_ternary_exact(dims, dtype, mode):
    _flush(f"gen ternary {dtype} {mode} dims={dims}")
    A, Bs = _inputs(dtype, 2, 300, dims, dist="ternary", seed=0x5EED0101)
    got, _ = _run(dtype, A, Bs, remap=mode)
    ref = oracle.cascade(dtype, A, Bs)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


# the configurations' widths on the 32x32x16 path (fewer rows and batches)
@pytest.mark.parametrize("mode", ["relabel", "permlane"])
@pytest.mark.parametrize("cfg,M,batch", [(1, 128, 1), (2, 1000, 3), (5, 700, 2)])
def test_configs_on_32x32(cfg, M, batch, mode):
    c = synth.WORKLOADS[cfg]
    _flush(f"gen forced cfg{cfg} {mode} M={M} batch={batch}")
    A, Bs = synth.make_inputs(cfg, M=M, batch=batch)
    got, info = _run(c["dtype"], A, Bs, remap=mode, mfma32=True)
    assert "mfma=32x32x16" in info, info
    assert_close(c["dtype"], got, oracle.cascade(c["dtype"], A, Bs), f"cfg{cfg} 32x32 {mode}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("dims", [(96, 160, 64), (64, 192, 96, 32)])
def test_unfused_matches_fused_bitwise(dims, dtype):
    """Lane-half swaps keep the natural K order, so the fused kernel and the
    per-GEMM kernels (intermediates rounded into HBM) feed the same values to
    the same instructions: the results agree bit for bit."""
    _flush(f"gen unfused vs fused {dtype} dims={dims}")
    A, Bs = _inputs(dtype, 2, 300, dims)
    fused, _ = _run(dtype, A, Bs, remap="permlane", mfma32=True)
    unf, info = _run(dtype, A, Bs, unfused=True, mfma32=True)
    assert "path=unfused" in info and "mfma=32x32x16" in info, info
    assert np.array_equal(fused, unf), f"{int((fused != unf).sum())} elements differ"
    assert_close(dtype, unf, oracle.cascade(dtype, A, Bs), "unfused 32x32")


def test_unfused_beyond_lds():
    """256 KB of weights do not fit the fused kernel's LDS, but one matrix at a
    time does: the unfused path covers the cascade."""
    dims = (256, 256, 256)
    _flush(f"gen unfused only dims={dims}")
    A, Bs = _inputs("f16", 1, 300, dims)
    with pytest.raises(cf.B2BError):
        cf.Plan("f16", 1, 300, *dims, mfma32=True)
    got, info = _run("f16", A, Bs, unfused=True, mfma32=True)
    assert "launches=2" in info, info
    assert_close("f16", got, oracle.cascade("f16", A, Bs), "unfused 256")


def _padded(x_dev, batch, rows, cols, ld, stride, fill):
    n = (batch - 1) * stride + rows * ld + 64
    buf = torch.full((n,), fill, dtype=x_dev.dtype, device="cuda")
    buf.as_strided((batch, rows, cols), (stride, ld, 1)).copy_(x_dev)
    return buf


@pytest.mark.parametrize("dims", [(96, 160, 64), (64, 192, 96, 32)])
def test_padded_and_broadcast(dims):
    dt, M, batch = "bf16", 300, 3
    _flush(f"gen strided dims={dims}")
    A, Bs = _inputs(dt, batch, M, dims)
    Bs = [b.copy() for b in Bs]
    Bs[0][:] = Bs[0][0]                       # B0 broadcast to every batch
    nst = len(dims) - 1
    lda, ldd = dims[0] + 8, dims[-1] + 16
    ldb = [dims[s + 1] + 8 * (s + 1) for s in range(nst)]
    sA, sD = M * lda + 8, M * ldd + 24
    sB = [0] + [dims[s] * ldb[s] + 8 for s in range(1, nst)]
    fill = float("nan")
    Ad = _padded(cf.to_device(A, dt), batch, M, dims[0], lda, sA, fill)
    Bd = [_padded(cf.to_device(Bs[0][:1], dt), 1, dims[0], dims[1], ldb[0], 0, fill)]
    Bd += [_padded(cf.to_device(Bs[s], dt), batch, dims[s], dims[s + 1], ldb[s], sB[s], fill)
           for s in range(1, nst)]
    Dd = torch.full(((batch - 1) * sD + M * ldd + 64,), fill, dtype=Ad.dtype, device="cuda")
    ld = [lda, ldb[0], ldb[1], ldb[2] if nst == 3 else 0, ldd]
    bs = [sA, sB[0], sB[1], sB[2] if nst == 3 else 0, sD]
    p = cf.Plan(dt, batch, M, *dims[:3], dims[3] if nst == 3 else 0, ld=ld, batch_stride=bs)
    assert "mfma=32x32x16" in p.info()
    p.run(Ad, *Bd, D=Dd)
    torch.cuda.synchronize()
    p.close()
    view = Dd.as_strided((batch, M, dims[-1]), (sD, ldd, 1))
    got = cf.to_host(view.contiguous())
    assert_close(dt, got, oracle.cascade(dt, A, Bs), f"gen strided {dims}")
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, dims[-1]), (sD, ldd, 1)).fill_(False)
    assert torch.isnan(Dd[mask]).all().item(), "writes outside the output windows"
