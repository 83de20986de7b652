"""GPU checks of b2b_gemm_tune: it keeps one of the compiled kernels for the
cascade (within the plan's flags), leaves D as that kernel computes it, and
the plan then runs that kernel with results within the tolerance."""
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


@pytest.mark.parametrize("cfg,M,batch,kw,expect", [
    (2, 2048, 4, dict(), None),                               # 16x16x32 modes and 32x32x16
    (5, 1024, 2, dict(), None),
    (4, 1024, 2, dict(), "f64_16x16x4"),
    (2, 1024, 2, dict(mfma32=True), "32x32x16"),              # only the 32x32x16 kernels
    (2, 1024, 2, dict(remap="bpermute"), "16x16x32"),         # only coordination rounds
])
def test_tune(cfg, M, batch, kw, expect):
    c = synth.CONFIGS[cfg]
    dt, dims = c["dtype"], c["dims"]
    _flush(f"tune cfg{cfg} M={M} batch={batch} {kw}")
    A, Bs = synth.make_inputs(cfg, M=M, batch=batch)
    Ad = cf.to_device(A, dt)
    Bd = [cf.to_device(b, dt) for b in Bs]
    p = cf.Plan(dt, batch, M, *dims[:3], dims[3] if len(dims) > 3 else 0, **kw)
    D = nan_output(dt, batch, M, dims[-1])
    p.tune([(Ad, Bd, D)], reps=3)
    info = p.info()
    if expect:
        assert f"mfma={expect}" in info, info
    if kw.get("remap") == "bpermute":
        assert "remap=bpermute" in info, info
    ref = oracle.cascade(dt, A, Bs)
    tuned = cf.to_host(D)
    assert_close(dt, tuned, ref, f"tune cfg{cfg}")
    D2 = nan_output(dt, batch, M, dims[-1])
    p.run(Ad, *Bd, D=D2)
    torch.cuda.synchronize()
    p.close()
    assert np.array_equal(cf.to_host(D2), tuned), "the plan runs the kernel the tuning kept"
