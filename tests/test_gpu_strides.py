"""GPU parity with non-dense layouts: padded leading dimensions, gaps between
batches and a weight broadcast to every batch (batch stride 0), for every
kernel family.  Padding elements of D must stay untouched."""
import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close

pytestmark = pytest.mark.gpu

ELT = {"f16": 2, "bf16": 2, "f64": 8}


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def _padded(x_dev, batch, rows, cols, ld, stride, fill):
    """Device buffer holding x (batch, rows, cols) at leading dimension ld and
    batch stride `stride` (elements); everything else set to `fill`."""
    n = (batch - 1) * stride + rows * ld + 64
    buf = torch.full((n,), fill, dtype=x_dev.dtype, device="cuda")
    buf.as_strided((batch, rows, cols), (stride, ld, 1)).copy_(x_dev)
    return buf


CASES = {
    # cfg: (M, batch) -- ragged M, several tiles
    2: (300, 3),     # fused, 128-wide fp16
    3: (200, 2),     # column-split, 256-wide bf16
    4: (300, 2),     # fused fp64
    5: (300, 2),     # three-GEMM fp16
}


@pytest.mark.parametrize("cfg", sorted(CASES))
def test_padded_and_broadcast(cfg):
    c = synth.WORKLOADS[cfg]
    dt, dims = c["dtype"], c["dims"]
    M, batch = CASES[cfg]
    _flush(f"strided cfg{cfg} M={M} batch={batch} dims={dims}")
    A, Bs = synth.make_inputs(cfg, M=M, batch=batch)
    Bs = [b.copy() for b in Bs]
    Bs[0][:] = Bs[0][0]                       # B0 broadcast: one matrix for every batch
    pad = 16 // ELT[dt]                       # one 16-byte step of padding
    K = dims[0]
    nst = len(dims) - 1
    lda, ldd = K + pad, dims[-1] + 2 * pad
    ldb = [dims[s + 1] + pad * (s + 1) for s in range(nst)]
    sA, sD = M * lda + pad, M * ldd + 3 * pad
    sB = [0] + [dims[s] * ldb[s] + pad for s in range(1, nst)]

    fill = float("nan")
    Ad = _padded(cf.to_device(A, dt), batch, M, K, lda, sA, fill)
    Bd = [_padded(cf.to_device(Bs[0][:1], dt), 1, dims[0], dims[1], ldb[0], 0, fill)]
    Bd += [_padded(cf.to_device(Bs[s], dt), batch, dims[s], dims[s + 1], ldb[s], sB[s], fill)
           for s in range(1, nst)]
    Dd = torch.full(((batch - 1) * sD + M * ldd + 64,), fill, dtype=Ad.dtype, device="cuda")

    ld = [lda, ldb[0], ldb[1], ldb[2] if nst == 3 else 0, ldd]
    bs = [sA, sB[0], sB[1], sB[2] if nst == 3 else 0, sD]
    p = cf.Plan(dt, batch, M, *dims[:3], dims[3] if nst == 3 else 0, ld=ld, batch_stride=bs)
    p.run(Ad, *Bd, D=Dd)
    torch.cuda.synchronize()
    p.close()

    view = Dd.as_strided((batch, M, dims[-1]), (sD, ldd, 1))
    got = cf.to_host(view.contiguous())
    ref = oracle.cascade(dt, A, Bs)
    assert_close(dt, got, ref, f"strided cfg{cfg}")
    # nothing outside the M x N windows was written
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, dims[-1]), (sD, ldd, 1)).fill_(False)
    assert torch.isnan(Dd[mask]).all().item(), "writes outside the output windows"
