"""The binding refuses tensors that do not fit a plan before anything is
launched (CPU): the kernels address memory by the plan's sizes, leading
dimensions and batch strides, so a tensor of another type, a smaller one or
one in host memory would be read or written out of bounds."""
import pytest
import torch

import chip_fusion_amd as cf


def _t(shape, dtype=torch.float16):
    return torch.zeros(shape, dtype=dtype)


def test_plan_run_checks_dtype_size_and_device():
    p = cf.Plan("f16", 2, 100, 64, 64, 64)
    A, B, D = _t((2, 100, 64)), _t((2, 64, 64)), _t((2, 100, 64))
    with pytest.raises(ValueError, match="A: dtype"):
        p.run(A.float(), B, B, D=D)
    with pytest.raises(ValueError, match="A: the plan addresses 12800 elements"):
        p.run(_t((2, 99, 64)), B, B, D=D)
    with pytest.raises(ValueError, match="B1: the plan addresses"):
        p.run(A, B, _t((1, 64, 64)), D=D)
    with pytest.raises(ValueError, match="D: dtype"):
        p.run(A, B, B, D=D.to(torch.bfloat16))
    # a view that starts inside its storage has fewer elements after it
    with pytest.raises(ValueError, match="A: the plan addresses"):
        p.run(_t((2 * 100 * 64 + 8,))[16:], B, B, D=D)
    with pytest.raises(ValueError, match="2 weight matrices expected, got 3"):
        p.run(A, B, B, B, D=D)
    # everything fits, but in host memory
    with pytest.raises(ValueError, match="device"):
        p.run(A, B, B, D=D)
    p.close()


def test_padded_and_broadcast_layouts():
    # lda 72, ldd 80, B1 broadcast (stride 0), batch gaps on D
    p = cf.Plan("f16", 3, 50, 64, 64, 64, ld=[72, 64, 64, 0, 80], batch_stride=[50 * 72, 4096, 0, 0, 51 * 80])
    A = _t((3 * 50 * 72,))
    B0, B1 = _t((3, 64, 64)), _t((64, 64))
    need_d = 2 * 51 * 80 + 49 * 80 + 64
    with pytest.raises(ValueError, match=f"D: the plan addresses {need_d}"):
        p.run(A, B0, B1, D=_t((need_d - 1,)))
    with pytest.raises(ValueError, match="device"):       # sizes fit: only the device is wrong
        p.run(A, B0, B1, D=_t((need_d,)))
    p.close()


def test_chain_types_and_tune_sets():
    p = cf.Chain(["f16", "fp8", "f16"], 1, 64, [64, 64, 32])
    A, B0, D = _t((1, 64, 64)), _t((1, 64, 64)), _t((1, 64, 32))
    with pytest.raises(ValueError, match="B1: dtype torch.uint8"):
        p.run(A, B0, _t((1, 64, 32)), D=D)
    with pytest.raises(ValueError, match="device"):
        p.run(A, B0, torch.zeros((1, 64, 32), dtype=torch.uint8), D=D)
    p.close()
    q = cf.Plan("f64", 1, 64, 64, 64, 64)
    Af, Bf = torch.zeros((1, 64, 64), dtype=torch.float64), torch.zeros((1, 64, 64), dtype=torch.float64)
    with pytest.raises(ValueError, match="D: the plan addresses"):
        q.tune([(Af, [Bf, Bf], torch.zeros((1, 63, 64), dtype=torch.float64))])
    q.close()


def test_probe_bindings_refuse_host_and_short_tensors():
    """The layout, rearrangement and round-executor probes read fixed sizes
    (16 bytes a lane, 8 for fp64, 32 for fp8; 64 * E words); tensors in host
    memory, or ones that do not hold those sizes, are refused first."""
    with pytest.raises(ValueError, match="device"):
        cf.mfma_probe("f16_16x16x32", _t((64, 8)), _t((64, 8)))
    with pytest.raises(ValueError, match="device"):
        cf.remap_probe("f16_16x16x32", "relabel", _t((512,), torch.int16))
    with pytest.raises(ValueError, match="device"):
        cf.remap_execute([[0] * 64], [[0] * 64], [[0] * 64], torch.zeros(64, dtype=torch.int32))
    with pytest.raises(ValueError, match="64 \\* E"):
        cf.remap_execute([[0] * 64], [[0] * 64], [[0] * 64], torch.zeros(32, dtype=torch.int32))
    with pytest.raises(ValueError, match=r"\[E, 64\]"):
        cf.remap_execute([[0] * 64], [[0] * 63], [[0] * 64], torch.zeros(64, dtype=torch.int32))
