"""Ragged and tiny M (fewer rows than one wave's 32, one either side of a
wave and of a workgroup tile, batches that straddle workgroup ranges) for the
tf32, per-stage-type and fp8-second-GEMM kernels, against the oracle."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close, nan_output

pytestmark = pytest.mark.gpu

SIZES = [(1, 1), (3, 31), (1, 33), (2, 255), (5, 257), (3, 129)]
KINDS = [
    ("tf32", ("tf32", "tf32", "tf32"), (64, 128, 32)),
    ("tf32-3", ("tf32", "tf32", "tf32", "tf32"), (32, 64, 96, 32)),
    ("typed", ("bf16", "f16", "bf16"), (96, 64, 128)),
    ("fp8", ("f16", "fp8", "f16"), (64, 128, 64)),
]


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("kind", range(len(KINDS)))
@pytest.mark.parametrize("size", SIZES)
def test_edges(kind, size):
    name, types, widths = KINDS[kind]
    batch, M = size
    _flush(f"edges {name} batch={batch} M={M} widths={widths}")
    seed = 0x5EED0700 + 17 * kind + M
    A = synth.tensor(seed, 0, (batch, M, widths[0]), types[0], "normal")
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), types[s], "normal", 1.0 / math.sqrt(widths[s]))
          for s in range(len(widths) - 1)]
    if name.startswith("tf32"):
        Ad = torch.from_numpy(A).cuda()
        Bd = [torch.from_numpy(b).cuda() for b in Bs]
        D = torch.full((batch, M, widths[-1]), float("nan"), dtype=torch.float32, device="cuda")
        p = cf.Chain("tf32", batch, M, list(widths))
    else:
        Ad = cf.to_device(A, types[0])
        Bd = [cf.to_device(b, types[s]) for s, b in enumerate(Bs)]
        D = nan_output(types[-1], batch, M, widths[-1])
        p = cf.Chain(list(types), batch, M, list(widths))
    p.run(Ad, *Bd, D=D)
    torch.cuda.synchronize()
    p.close()
    got = cf.to_host(D)
    if name.startswith("tf32"):
        ref = oracle.cascade("tf32", A, Bs).astype(np.float64)
        g = got.astype(np.float64)
        assert np.all(np.isfinite(g))
        assert np.linalg.norm(g - ref) / np.linalg.norm(ref) <= 1e-3
    else:
        assert_close(types[-1], got, oracle.cascade(list(types), A, Bs), f"{name} M={M}")
