"""Error paths on the GPU, forced from the host: an unfused plan whose
workspace allocation fails (B2B_FAULT_INJECT=alloc[:N], the library's test
hook) returns OUT_OF_MEMORY, leaves *plan NULL and frees what it had already
allocated.  No kernel runs."""
import ctypes

import pytest
import torch

import chip_fusion_amd as cf

pytestmark = pytest.mark.gpu

# three GEMMs unfused: two intermediates of 64 x 4096 x 128 fp16 = 64 MiB each
SHAPE = dict(dtype=0, batch=64, M=4096, K=128, N1=128, N2=128, N3=128)


def _create_unfused():
    h = ctypes.c_void_p(123)
    s = SHAPE
    st = cf.lib().b2b_gemm_create(ctypes.byref(h), s["dtype"], s["batch"], s["M"], s["K"], s["N1"], s["N2"],
                                  s["N3"], None, None, cf.FLAG_UNFUSED)
    return st, h


def _free():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_unfused_workspace_allocation_failure(monkeypatch):
    print("\n[case] unfused workspace allocation failure", flush=True)
    st, h = _create_unfused()                       # the same plan allocates without the hook
    assert st == 0 and h.value
    buf = ctypes.create_string_buffer(512)
    assert cf.lib().b2b_gemm_get_info(h, buf, 512) == 0
    assert "workspace_bytes=134217728" in buf.value.decode()
    assert cf.lib().b2b_gemm_destroy(h) == 0
    free0 = _free()
    for spec in ["alloc", "alloc:1"] + ["alloc:2"] * 10:
        monkeypatch.setenv("B2B_FAULT_INJECT", spec)
        st, h = _create_unfused()
        assert st == 4, spec                         # B2B_ERROR_OUT_OF_MEMORY
        assert h.value is None, spec
    # the ten failures at the second allocation each had 64 MiB from the first:
    # all of it was returned
    assert free0 - _free() < 32 << 20
    monkeypatch.setenv("B2B_FAULT_INJECT", "alloc:3")  # past the plan's two allocations: no effect
    st, h = _create_unfused()
    assert st == 0 and h.value
    cf.lib().b2b_gemm_destroy(h)
