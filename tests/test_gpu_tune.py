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
    c = synth.WORKLOADS[cfg]
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


@pytest.mark.parametrize("types,widths", [(("f16", "bf16", "f16"), (128, 128, 128)),
                                          (("f16", "fp8", "f16"), (128, 128, 128)),
                                          # wider than the 128-bound fp8 instances: only the
                                          # 256-bound ones may compete (a narrower one would
                                          # walk only part of K and of D's columns)
                                          (("f16", "fp8", "f16"), (256, 128, 128)),
                                          (("bf16", "fp8", "bf16"), (128, 128, 256)),
                                          # compiled masks and the run-time-typed instance compete
                                          (("f16", "bf16", "f16", "bf16"), (128, 128, 128, 64)),
                                          (("tf32", "tf32", "tf32"), (128, 128, 64))])
def test_tune_typed_fp8_tf32(types, widths):
    """Tuning a plan with a type per stage, an fp8 second GEMM or tf32 keeps a
    kernel of that same kind (the instances differ only in waves per
    workgroup); its result is within the tolerance and the plan then
    reproduces it."""
    M, batch = 1024, 2
    _flush(f"tune {types} {widths}")
    if types[0] == "tf32":
        A = synth.tensor(5, 0, (batch, M, widths[0]), "tf32", "normal")
        Bs = [synth.tensor(5, 1 + s, (batch, widths[s], widths[s + 1]), "tf32", "normal", widths[s] ** -0.5)
              for s in range(len(widths) - 1)]
        p = cf.Chain("tf32", batch, M, list(widths))
        Ad = torch.from_numpy(A).cuda()
        Bd = [torch.from_numpy(b).cuda() for b in Bs]
        D = torch.full((batch, M, widths[-1]), float("nan"), dtype=torch.float32, device="cuda")
    else:
        A = synth.tensor(5, 0, (batch, M, widths[0]), types[0], "normal")
        Bs = [synth.tensor(5, 1 + s, (batch, widths[s], widths[s + 1]), types[s], "normal", widths[s] ** -0.5)
              for s in range(len(widths) - 1)]
        p = cf.Chain(list(types), batch, M, list(widths))
        Ad = cf.to_device(A, types[0])
        Bd = [cf.to_device(b, types[s]) for s, b in enumerate(Bs)]
        D = nan_output(types[-1], batch, M, widths[-1])
    kind = lambda info: {k: v for k, v in (kv.split("=", 1) for kv in info.split())
                         if k in ("path", "dtype", "mfma", "remap", "dims")}
    before = kind(p.info())
    p.tune([(Ad, Bd, D)], reps=3)
    assert kind(p.info()) == before, (before, p.info())    # a kernel of the same kind (any wave count)
    tuned = cf.to_host(D)
    if types[0] == "tf32":
        ref = oracle.cascade("tf32", A, Bs).astype(np.float64)
        assert np.linalg.norm(tuned - ref) / np.linalg.norm(ref) < 1e-3
    else:
        assert_close(types[-1], tuned, oracle.cascade(list(types), A, Bs), f"tune {types}")
    D2 = torch.full_like(D, float("nan"))
    p.run(Ad, *Bd, D=D2)
    torch.cuda.synchronize()
    p.close()
    assert np.array_equal(cf.to_host(D2), tuned)
