"""K and N tails: widths that are not multiples of the instruction granule
(32 for fp16/bf16; 8 for fp64's K and 16 for its N), rows at any element
alignment (dense rows of such widths, or padded leading dimensions that are
not 16-byte multiples), batch gaps and a broadcast weight -- fused and
unfused, against the oracle.  The cascade is defined for any widths; the
kernels pad every width on chip with zeros, which changes no sum, so
small-integer (ternary) inputs must match bit for bit, Gaussian ones within
the tolerance.  Nothing outside D's M x N windows may be written."""
import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(dtype, batch, M, widths, dist, seed):
    scale = lambda d: 1.0 if dist != "normal" else d ** -0.5
    A = synth.tensor(seed, 0, (batch, M, widths[0]), dtype, dist, 1.0)
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), dtype, dist, scale(widths[s]))
          for s in range(len(widths) - 1)]
    return A, Bs


def _place(x_host, dtype, batch, rows, cols, ld, stride, fill):
    """Device buffer holding x (batch, rows, cols) at leading dimension ld and
    batch stride `stride` (elements); every other element is `fill`."""
    dev = cf.to_device(x_host, dtype)
    n = max(1, (batch - 1) * stride + (rows - 1) * ld + cols) + 37
    buf = torch.full((n,), fill, dtype=dev.dtype, device="cuda")
    buf.as_strided((batch, rows, cols), (stride, ld, 1)).copy_(dev.reshape(batch, rows, cols))
    return buf


def _run(dtype, batch, M, widths, A, Bs, ld=None, bs=None, unfused=False, broadcast0=False):
    """Runs the cascade through the C ABI with the given layout; returns D's
    host encodings (batch, M, N) and whether anything outside D's windows
    changed."""
    nst = len(widths) - 1
    L = ld or [widths[0]] + list(widths[1:]) + [widths[-1]]
    rows = [M] + list(widths[:-1]) + [M]
    S = bs or [r * l for r, l in zip(rows, L)]
    nan = float("nan")
    Ad = _place(A, dtype, batch, M, widths[0], L[0], S[0], nan)
    Bd = []
    for s in range(nst):
        if s == 0 and broadcast0:
            Bd.append(_place(Bs[0][:1], dtype, 1, widths[0], widths[1], L[1], 0, nan))
        else:
            Bd.append(_place(Bs[s], dtype, batch, widths[s], widths[s + 1], L[1 + s], S[1 + s], nan))
    tdt = cf.TORCH_DTYPES[cf.DTYPES[dtype]]
    nD = (batch - 1) * S[-1] + (M - 1) * L[-1] + widths[-1] + 41
    Dd = torch.full((nD,), nan, dtype=tdt, device="cuda")
    p = cf.Chain(dtype, batch, M, list(widths), ld=L, batch_stride=S, unfused=unfused)
    info = p.info()
    p.run(Ad, *Bd, D=Dd)
    torch.cuda.synchronize()
    p.close()
    view = Dd.as_strided((batch, M, widths[-1]), (S[-1], L[-1], 1))
    got = cf.to_host(view.contiguous())
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, widths[-1]), (S[-1], L[-1], 1)).fill_(False)
    untouched = torch.isnan(Dd[mask]).all().item()
    return got, untouched, info


# (dtype, batch, M, widths): fused on the tail kernels
FUSED = [
    ("f16", 2, 300, [100, 72, 50]),
    ("bf16", 3, 77, [100, 72, 50]),
    ("f16", 2, 300, [100, 72, 50, 40]),
    ("f16", 1, 33, [1, 1, 1]),
    ("bf16", 2, 257, [31, 33, 7]),
    ("f16", 1, 513, [250, 150, 130]),             # 256-wide bound
    ("bf16", 2, 129, [200, 17, 250, 3]),          # three GEMMs, 256-wide bound
    ("f64", 3, 129, [10, 20, 36]),
    ("f64", 2, 100, [10, 20, 36, 12]),
    ("f64", 2, 300, [3, 5, 7]),
    ("f64", 1, 129, [64, 17, 63]),
]


@pytest.mark.parametrize("dtype,batch,M,widths", FUSED)
@pytest.mark.parametrize("dist", ["normal", "ternary"])
def test_tails_fused_dense(dtype, batch, M, widths, dist):
    """Dense rows of tail widths (rows at any element alignment)."""
    _flush(f"tails fused {dtype} b{batch} M{M} {widths} {dist}")
    A, Bs = _inputs(dtype, batch, M, widths, dist, 0x7A11 + M)
    got, untouched, info = _run(dtype, batch, M, widths, A, Bs)
    assert "path=fused" in info and "tail=1" in info, info
    ref = oracle.cascade(dtype, A, Bs)
    if dist == "ternary":
        assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"
    else:
        assert_close(dtype, got, ref, f"tails {dtype} {widths}")
    assert untouched, "writes outside D's windows"


# padded leading dimensions (not 16-byte multiples), batch gaps, B0 broadcast
STRIDED = [
    ("f16", 3, 300, [100, 72, 50]),
    ("bf16", 2, 129, [64, 96, 32]),               # whole granules, rows off 16-byte boundaries
    ("f16", 2, 77, [31, 33, 7, 45]),
    ("f64", 3, 129, [10, 20, 36]),
    ("f64", 2, 100, [16, 32, 48]),                # whole granules, odd leading dimensions
]


@pytest.mark.parametrize("dtype,batch,M,widths", STRIDED)
def test_tails_padded_and_broadcast(dtype, batch, M, widths):
    _flush(f"tails strided {dtype} b{batch} M{M} {widths}")
    A, Bs = _inputs(dtype, batch, M, widths, "normal", 0x57D + M)
    Bs = [b.copy() for b in Bs]
    Bs[0][:] = Bs[0][0]                            # one B0 for every batch
    nst = len(widths) - 1
    L = [widths[0] + 3] + [widths[s + 1] + 1 + s for s in range(nst)] + [widths[-1] + 5]
    rows = [M] + list(widths[:-1]) + [M]
    S = [rows[0] * L[0] + 7, 0] + [rows[1 + s] * L[1 + s] + 3 for s in range(1, nst)] + [M * L[-1] + 9]
    got, untouched, info = _run(dtype, batch, M, widths, A, Bs, ld=L, bs=S, broadcast0=True)
    assert "tail=1" in info, info
    assert_close(dtype, got, oracle.cascade(dtype, A, Bs), f"tails strided {dtype} {widths}")
    assert untouched, "writes outside D's windows"


# unfused: one tail kernel per GEMM (fp64 past the fused bound of 64)
UNFUSED = [
    ("f16", 2, 300, [100, 72, 50]),
    ("bf16", 1, 129, [250, 200, 130, 5]),         # too wide for one fused kernel's LDS
    ("f64", 2, 129, [100, 1, 100]),
    ("f64", 1, 77, [10, 20, 36, 12]),
]


@pytest.mark.parametrize("dtype,batch,M,widths", UNFUSED)
@pytest.mark.parametrize("dist", ["normal", "ternary"])
def test_tails_unfused(dtype, batch, M, widths, dist):
    _flush(f"tails unfused {dtype} b{batch} M{M} {widths} {dist}")
    A, Bs = _inputs(dtype, batch, M, widths, dist, 0xF00 + M)
    got, untouched, info = _run(dtype, batch, M, widths, A, Bs, unfused=True)
    assert "path=unfused" in info, info
    ref = oracle.cascade(dtype, A, Bs)
    if dist == "ternary":
        assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"
    else:
        assert_close(dtype, got, ref, f"tails unfused {dtype} {widths}")
    assert untouched, "writes outside D's windows"


def test_tails_static_workspace():
    """The allocation-free unfused entry point takes tails too."""
    _flush("tails static workspace")
    dtype, batch, M, widths = "f16", 2, 300, [100, 72, 50, 40]
    A, Bs = _inputs(dtype, batch, M, widths, "ternary", 0x5747)
    Ad = cf.to_device(A, dtype)
    Bd = [cf.to_device(b, dtype) for b in Bs]
    D = torch.full((batch, M, widths[-1]), float("nan"), dtype=torch.float16, device="cuda")
    cf.chain_run_static(dtype, batch, M, widths, Ad, Bd, D)
    torch.cuda.synchronize()
    assert np.array_equal(cf.to_host(D), oracle.cascade(dtype, A, Bs))
