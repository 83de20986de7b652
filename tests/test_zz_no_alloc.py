"""b2b_chain_run_static -- the unfused cascade with the library's static
device workspace, for callers that cannot allocate -- against the unfused
plan (b2b_chain_create with B2B_FLAG_UNFUSED, then b2b_chain_run), which runs
the same single-GEMM kernels in the same order: D must agree bit for bit, on
two calls in a row, the second smaller than the first (the workspace keeps
the first call's intermediates; nothing may read them)."""
import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import synth

pytestmark = pytest.mark.gpu

# (dtype, [(batch, M, widths), ...]) -- each list: two calls in a row, the second smaller
CASES = [
    ("f16", [(2, 1000, [128, 128, 128, 64]), (1, 300, [64, 64, 64, 32])]),
    ("bf16", [(1, 4096, [256, 256, 256]), (3, 77, [32, 96, 64])]),
    ("f64", [(2, 2048, [64, 64, 64, 64]), (1, 129, [16, 32, 48])]),
    ("f16", [(1, 2048, [96, 160, 64, 32, 128]), (2, 513, [64, 64])]),   # four GEMMs, then one
]


def _inputs(dtype, batch, M, widths, seed):
    A = synth.tensor(seed, 0, (batch, M, widths[0]), dtype, "normal")
    Bs = [synth.tensor(seed, 1 + s, (batch, widths[s], widths[s + 1]), dtype, "normal", widths[s] ** -0.5)
          for s in range(len(widths) - 1)]
    return cf.to_device(A, dtype), [cf.to_device(b, dtype) for b in Bs]


@pytest.mark.parametrize("dtype,calls", CASES)
def test_static_workspace_matches_unfused_plan(dtype, calls):
    for i, (batch, M, widths) in enumerate(calls):
        print(f"\n[case] static workspace {dtype} call {i}: batch={batch} M={M} widths={widths}", flush=True)
        A, Bs = _inputs(dtype, batch, M, widths, 0x5A7E0000 + i)
        tdt = cf.TORCH_DTYPES[cf.DTYPES[dtype]]
        ref = torch.full((batch, M, widths[-1]), float("nan"), dtype=tdt, device="cuda")
        plan = cf.Chain(dtype, batch, M, widths, unfused=True)
        plan.run(A, *Bs, D=ref)
        got = torch.full_like(ref, float("nan"))
        cf.chain_run_static(dtype, batch, M, widths, A, Bs, got)
        torch.cuda.synchronize()
        plan.close()
        r, g = cf.to_host(ref), cf.to_host(got)
        assert np.all(np.isfinite(cf.to_host(got.float() if dtype != "f64" else got))), "unwritten output"
        assert np.array_equal(g, r), f"call {i}: {int((g != r).sum())} elements differ"


def test_static_workspace_padded_layout():
    """Leading dimensions and batch strides as for b2b_chain_create."""
    print("\n[case] static workspace padded layout", flush=True)
    batch, M, widths = 2, 300, [64, 96, 32]
    ld, bs = [72, 96, 40, 48], [300 * 72, 0, 96 * 40, 310 * 48]
    A = torch.randn(batch * 300 * 72, device="cuda").half()
    B0 = torch.randn(64 * 96, device="cuda").half() / 8
    B1 = torch.randn(batch * 96 * 40, device="cuda").half() / 8
    ref = torch.zeros(batch * 310 * 48, dtype=torch.float16, device="cuda")
    got = torch.zeros_like(ref)
    plan = cf.Chain("f16", batch, M, widths, ld=ld, batch_stride=bs, unfused=True)
    plan.run(A, B0, B1, D=ref)
    cf.chain_run_static("f16", batch, M, widths, A, [B0, B1], got, ld=ld, batch_stride=bs)
    torch.cuda.synchronize()
    plan.close()
    assert torch.equal(ref, got)
