"""Plan runs captured in a HIP graph (torch.cuda.CUDAGraph, which is a HIP
graph on ROCm): a run enqueues kernels only (no allocation, no memset), so
its capture replays.  Each case runs eagerly once (grid sizes and kernel
attributes are set up on first use), captures one run, then replays it three
times with new inputs copied into the captured buffers in between (eager work
and a synchronisation between replays); every replay must equal an eager run
on the same inputs bit for bit."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import synth

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


CASES = [
    ("fixed f16", "f16", (128, 128, 128), {}),
    ("32x32x16", "f16", (128, 96, 128), {"mfma32": True}),
    ("tf32", "tf32", (64, 128, 64), {}),
    ("typed", ["f16", "bf16", "f16"], (128, 128, 64), {}),
    ("typed, types read at run time", ["bf16", "f16", "f16", "bf16", "f16"], (64, 96, 64, 128, 64), {}),
    ("fp8 stage", ["f16", "fp8", "f16"], (64, 128, 64), {}),
    ("unfused", "bf16", (128, 128, 128), {"unfused": True}),
]


def _tensors(types, batch, M, widths, seed):
    A = synth.tensor(seed, 0, (batch, M, widths[0]), types[0], "normal")
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), types[s], "normal", widths[s] ** -0.5)
          for s in range(len(widths) - 1)]
    return cf.to_device(A, types[0]), [cf.to_device(b, types[s]) for s, b in enumerate(Bs)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_graph_replay(case):
    name, dtype, widths, kw = CASES[case]
    _flush(f"graph {name} widths={widths}")
    types = dtype if isinstance(dtype, list) else [dtype] * len(widths)
    batch, M = 2, 300
    plan = cf.Chain(dtype, batch, M, list(widths), **kw)
    A, Bs = _tensors(types, batch, M, widths, 0x5EED0800)
    D = torch.empty((batch, M, widths[-1]), dtype=cf.TORCH_DTYPES[cf.DTYPES[types[-1]]], device="cuda")
    plan.run(A, *Bs, D=D)                       # eager first: set-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            plan.run(A, *Bs, D=D, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        A2, Bs2 = _tensors(types, batch, M, widths, 0x5EED0810 + rep)
        A.copy_(A2)
        for b, b2 in zip(Bs, Bs2):
            b.copy_(b2)
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = cf.to_host(D)
        Dref = torch.full_like(D, float("nan"))
        plan.run(A2, *Bs2, D=Dref)
        torch.cuda.synchronize()
        want = cf.to_host(Dref)
        assert np.array_equal(got, want), f"replay {rep}: {int((got != want).sum())} elements differ"
    plan.close()


def test_one_plan_on_two_streams():
    """A fused plan holds no device memory: one plan enqueued on two streams
    at once, on different inputs, gives each stream's result exactly."""
    _flush("one plan, two streams")
    batch, M, widths = 4, 2048, (128, 128, 128)
    plan = cf.Chain("f16", batch, M, list(widths))
    sets = [_tensors(["f16"] * 3, batch, M, widths, 0x5EED0820 + i) for i in range(2)]
    want = []
    for A, Bs in sets:
        D = torch.empty((batch, M, widths[-1]), dtype=torch.float16, device="cuda")
        plan.run(A, *Bs, D=D)
        torch.cuda.synchronize()
        want.append(cf.to_host(D))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((batch, M, widths[-1]), float("nan"), dtype=torch.float16, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(5):
        for (A, Bs), D, s in zip(sets, outs, streams):
            plan.run(A, *Bs, D=D, stream=s)
    torch.cuda.synchronize()
    for D, w in zip(outs, want):
        assert np.array_equal(cf.to_host(D), w)
    plan.close()
