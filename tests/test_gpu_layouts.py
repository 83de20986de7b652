"""The layout catalogue on the hardware: one matrix instruction with operands
placed by the assumed A/B layouts must give, read through the assumed
accumulator layout, exactly the product of the two integer matrices."""
import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
from oracle import remap as R

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", ["f16_16x16x32", "bf16_16x16x32", "f16_32x32x16", "bf16_32x32x16",
                                   "f64_16x16x4"])
def test_mfma_layout(shape):
    sh = R.SHAPES[shape]
    rng = np.random.default_rng(1)
    A = rng.integers(-3, 4, (sh.m, sh.k)).astype(np.float64)
    B = rng.integers(-3, 4, (sh.k, sh.n)).astype(np.float64)
    # make every output distinct so a misplaced lane/register is identifiable
    A[:, 0] = np.arange(sh.m) + 1
    B[0, :] = 100.0
    if sh.k > 1:
        A[:, 1] = 1.0
        B[1, :] = np.arange(sh.n) + 1
    C = A @ B
    a = np.zeros((64, sh.a_elems)); b = np.zeros((64, sh.a_elems))
    for l in range(64):
        for u in range(sh.a_elems):
            i, k = sh.a(l, u); a[l, u] = A[i, k]
            k, j = sh.b(l, u); b[l, u] = B[k, j]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}[shape.split("_")[0]]
    ad = torch.tensor(a, dtype=tdt, device="cuda").contiguous()
    bd = torch.tensor(b, dtype=tdt, device="cuda").contiguous()
    c = cf.mfma_probe(shape, ad, bd).cpu().double().numpy()
    torch.cuda.synchronize()
    want = np.zeros((64, sh.c_elems))
    for l in range(64):
        for v in range(sh.c_elems):
            i, j = sh.c(l, v); want[l, v] = C[i, j]
    if not np.array_equal(c, want):
        where = {}
        for i in range(sh.m):
            for j in range(sh.n):
                where.setdefault(C[i, j], []).append((i, j))
        found = [[where.get(c[l, v], "?") for v in range(sh.c_elems)] for l in (0, 1, 15, 16, 17, 31, 32, 48, 63)]
        pytest.fail(f"layout mismatch; lanes 0,1,15,16,17,31,32,48,63 hold (i,j) = {found}")
