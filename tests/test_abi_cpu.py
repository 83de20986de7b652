"""C ABI checks that need no GPU: the library loads and exports every symbol
the header declares, argument validation, and the host-side rearrangement
tables against the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import chip_fusion_amd as cf
from oracle import remap as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="b2b.h"):
    txt = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"\b(b2b_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = cf.lib()
    names = _declared()
    assert "b2b_gemm_create" in names and "b2b_gemm_run" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(cf.EXPORTS)
    bench = _declared("b2b_bench.h")
    for n in bench:
        assert hasattr(L, n), n
    assert set(bench) == set(cf.BENCH_EXPORTS)


def test_bench_instruments_reject_bad_arguments():
    """The measurement calls validate before launching (no GPU needed)."""
    L = cf.lib()
    flop = ctypes.c_double()
    p = ctypes.c_void_p(0x1000)
    assert L.b2b_bench_mfma(0, 0, 10, p, ctypes.byref(flop), None) == 1          # no workgroups
    assert L.b2b_bench_mfma(0, 4, 0, p, ctypes.byref(flop), None) == 1           # no rounds
    assert L.b2b_bench_mfma(0, 4, 10, None, ctypes.byref(flop), None) == 1       # no sink
    assert L.b2b_bench_mfma(3, 4, 10, p, ctypes.byref(flop), None) == 2          # tf32: no loop
    assert L.b2b_bench_copy(p, ctypes.c_void_p(0x100000), 100, 4, None) == 1     # not whole 64 bytes
    assert L.b2b_bench_copy(p, ctypes.c_void_p(0x1040), 128, 4, None) == 1       # overlapping
    assert L.b2b_bench_copy(ctypes.c_void_p(0x1008), ctypes.c_void_p(0x100000), 128, 4, None) == 1
    q = ctypes.c_void_p(0x100000)
    assert L.b2b_bench_stream(p, 256, q, 100, 4, None) == 1                      # not whole 64 bytes
    assert L.b2b_bench_stream(p, 192, q, 128, 4, None) == 1                      # not a whole ratio
    assert L.b2b_bench_stream(p, 640, q, 128, 4, None) == 1                      # ratio above 4
    assert L.b2b_bench_stream(p, 64, q, 128, 4, None) == 1                       # fewer bytes read than written
    assert L.b2b_bench_stream(p, 512, ctypes.c_void_p(0x1100), 128, 4, None) == 1   # dst inside src
    assert L.b2b_bench_stream(p, 256, q, 128, 0, None) == 1                      # no workgroups
    assert L.b2b_bench_stream(ctypes.c_void_p(0x1008), 256, q, 128, 4, None) == 1   # misaligned


def _create(**kw):
    args = dict(dtype=0, batch=1, M=128, K=64, N1=64, N2=64, N3=0, ld=None, bs=None, flags=0)
    args.update(kw)
    h = ctypes.c_void_p(123)
    arr = ctypes.c_int64 * 5
    st = cf.lib().b2b_gemm_create(ctypes.byref(h), args["dtype"], args["batch"], args["M"], args["K"],
                                  args["N1"], args["N2"], args["N3"],
                                  arr(*args["ld"]) if args["ld"] else None,
                                  arr(*args["bs"]) if args["bs"] else None, args["flags"])
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), 1), (dict(K=0), 1), (dict(N1=-1), 1), (dict(batch=0), 1), (dict(N3=-2), 1),
    (dict(dtype=7), 2),
    (dict(ld=[60, 64, 64, 0, 64]), 1),        # lda below K
    (dict(ld=[68, 64, 64, 0, 64], flags=1 << 4), 1),   # rows off 16-byte boundaries: only the
                                                        # tail kernels take them, and they relabel
    (dict(flags=1 << 12), 1),                 # unknown flag
    (dict(flags=(7 << 4)), 1),                # unknown remap mode
    (dict(flags=2 | (2 << 4)), 1),            # orientation N with permlane
    (dict(K=96, N1=80, N2=96, flags=2 | (1 << 4)), 2),  # a tail with orientation N
    (dict(K=80, N1=64, N2=64, flags=3 << 4), 2),        # a tail with the LDS rearrangement
    (dict(K=96, N1=96, N2=288), 2),           # a width above 256
    (dict(dtype=2, K=96, N1=96, N2=160), 2),  # fp64: widths above 128
    (dict(dtype=2, K=92, N1=96, N2=96), 2),   # fp64 tails fuse up to 64 wide (96 pads to 96)
    (dict(K=256, N1=256, N2=256, flags=4), 2),         # 32x32 path: 256 KB of weights
    (dict(dtype=2, flags=4), 2),                       # 32x32 path: 16-bit types only
    (dict(flags=4 | (1 << 4)), 2),                     # 32x32 path: no coordination rounds
    (dict(flags=4 | 2 | (3 << 4)), 2),                 # 32x32 path: orientation T only
    (dict(batch=2, bs=[0, 4096, 4096, 0, 8192]), 1),   # A broadcast over batches
    # 32-bit buffer offsets: 32 rows of A (or D), or a whole weight matrix,
    # must span less than 2^31 bytes
    (dict(ld=[1 << 25, 64, 64, 0, 64]), 1),            # 32 rows x 2^25 x 2 bytes = 2^31
    (dict(ld=[64, 64, 64, 0, 1 << 25]), 1),
    (dict(ld=[64, 1 << 24, 64, 0, 64]), 1),            # 64 rows of B0 x 2^24 x 2 bytes = 2^31
    (dict(dtype=2, ld=[1 << 23, 64, 64, 0, 64]), 1),   # fp64: 32 x 2^23 x 8 bytes
])
def test_create_rejects(kw, status):
    st, h = _create(**kw)
    assert st == status
    assert h.value is None


def test_create_accepts_and_destroy():
    st, h = _create()
    assert st == 0 and h.value
    buf = ctypes.create_string_buffer(256)
    assert cf.lib().b2b_gemm_get_info(h, buf, 256) == 0
    assert b"path=fused" in buf.value and b"remap=relabel" in buf.value
    assert cf.lib().b2b_gemm_destroy(h) == 0
    assert cf.lib().b2b_gemm_destroy(None) == 0


def _info(**kw):
    st, h = _create(**kw)
    assert st == 0 and h.value, st
    buf = ctypes.create_string_buffer(512)
    assert cf.lib().b2b_gemm_get_info(h, buf, 512) == 0
    assert cf.lib().b2b_gemm_destroy(h) == 0
    return dict(kv.split("=", 1) for kv in buf.value.decode().split())


@pytest.mark.parametrize("kw,expect", [
    # widths no fixed-width kernel covers go to the run-time-width kernels
    (dict(K=96, N1=160, N2=64), dict(path="fused", mfma="32x32x16", remap="relabel", lds_bytes=str(51200 + 32768))),
    (dict(dtype=1, K=32, N1=32, N2=256, N3=32), dict(mfma="32x32x16", dims="32x32x256x32")),
    (dict(K=96, N1=160, N2=64, flags=2 << 4), dict(mfma="32x32x16", remap="permlane")),
    # fp64 widths no fixed-width kernel covers: run-time widths on 16x16x4
    (dict(dtype=2, K=96, N1=48, N2=112), dict(mfma="f64_16x16x4", remap="relabel", rows_per_wg="128")),
    (dict(dtype=2, K=8, N1=128, N2=16, N3=64), dict(mfma="f64_16x16x4", dims="8x128x16x64")),
    # the configurations' widths keep their fixed-width kernels unless asked
    (dict(), dict(mfma="16x16x32", remap="relabel")),
    # four waves (two workgroups a CU): 4 x 4 KB of D staging
    (dict(flags=4), dict(mfma="32x32x16", remap="relabel", waves="4", lds_bytes=str(16384 + 16384))),
    (dict(K=128, N1=128, N2=128, N3=64, flags=4 | (2 << 4)), dict(mfma="32x32x16", remap="permlane")),
    # the 256-wide cascade (256 KB of weights) keeps its column-split kernel
    (dict(dtype=1, K=256, N1=256, N2=256), dict(mfma="16x16x32", remap="lds")),
])
def test_plan_selection(kw, expect):
    info = _info(**kw)
    for k, v in expect.items():
        assert info[k] == v, (k, info)


def test_run_rejects_bad_pointers():
    st, h = _create()
    assert st == 0
    L = cf.lib()
    a = ctypes.c_void_p(0x1000)
    assert L.b2b_gemm_run(None, a, a, a, None, ctypes.c_void_p(0x2000), None) == 1
    assert L.b2b_gemm_run(h, None, a, a, None, ctypes.c_void_p(0x2000), None) == 1
    assert L.b2b_gemm_run(h, a, a, a, a, ctypes.c_void_p(0x2000), None) == 1       # B2 with N3 == 0
    assert L.b2b_gemm_run(h, ctypes.c_void_p(0x1008), a, a, None, ctypes.c_void_p(0x2000), None) == 1
    assert L.b2b_gemm_run(h, a, a, a, None, a, None) == 1                           # D aliases A
    L.b2b_gemm_destroy(h)


def test_status_strings():
    for s in range(6):
        assert cf.lib().b2b_status_string(s).decode() == cf.STATUS[s]


SHAPES = ["f16_16x16x32", "bf16_16x16x32", "f16_32x32x16", "bf16_32x32x16", "f16_16x16x16",
          "f64_16x16x4"]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("orient", ["T", "N"])
def test_relation_tables_match_oracle(shape, orient):
    """The library's layout catalogue and relation builder against the oracle's
    independent enumeration, bit for bit."""
    rel, E = cf.remap_relation(shape, orient == "N")
    src, dst, meta = R.cascade_layouts(shape, orient)
    assert E == meta["elems"]
    assert np.array_equal(rel, np.array(R.relation(src, dst)))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("orient,packed", [("T", True), ("T", False), ("N", False)])
def test_schedules_valid_and_match_oracle(shape, orient, packed):
    if packed and shape.startswith("f64"):
        pytest.skip("fp64 elements are already 64-bit")
    src, dst, meta = R.cascade_layouts(shape, orient)
    rel = R.per_lane(R.relation(src, dst), 64, meta["elems"])
    if packed:
        rel = R.pack_pairs(rel)
    p, q, r = cf.remap_schedule(shape, orient == "N", packed)
    H = [[(int(p[j, i]), int(q[j, i]), int(r[j, i])) for j in range(p.shape[0])] for i in range(64)]
    ok, why = R.validate(H, rel)
    assert ok, why
    assert H == R.coordination_matrix(rel)


def test_build_rejects_scratch_spills():
    from chip_fusion_amd import build
    log = ("x.hpp:1:1: remark: Function Name: _ZN4b2bk12fused_kernelI1AEEvv [-Rpass-analysis]\n"
           "x.hpp:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis]\n"
           "x.hpp:1:1: remark: Function Name: _ZN4b2bk10gen_kernelI1BEEvv [-Rpass-analysis]\n"
           "x.hpp:1:1: remark:     ScratchSize [bytes/lane]: 80 [-Rpass-analysis]\n")
    assert build._scratch_kernels(log) == [("_ZN4b2bk10gen_kernelI1BEEvv", 80)]


def _chain(dtype=0, batch=1, M=128, widths=(128, 128, 128, 128, 64), ld=None, bs=None, flags=0, nst=None):
    h = ctypes.c_void_p(123)
    n = len(widths) - 1 if nst is None else nst
    w = (ctypes.c_int64 * len(widths))(*widths) if widths is not None else None
    arr = ctypes.c_int64 * (len(widths) + 1 if widths else 1)
    st = cf.lib().b2b_chain_create(ctypes.byref(h), dtype, batch, M, n, w,
                                   arr(*ld) if ld else None, arr(*bs) if bs else None, flags)
    return st, h


def _chain_info(**kw):
    st, h = _chain(**kw)
    assert st == 0 and h.value, st
    buf = ctypes.create_string_buffer(512)
    assert cf.lib().b2b_gemm_get_info(h, buf, 512) == 0
    assert cf.lib().b2b_gemm_destroy(h) == 0
    return dict(kv.split("=", 1) for kv in buf.value.decode().split())


@pytest.mark.parametrize("kw,status", [
    (dict(nst=0, widths=(128,)), 1),
    (dict(nst=9, widths=(64,) * 10), 1),
    (dict(widths=None, nst=2), 1),
    (dict(widths=(128, 0, 128)), 1),
    (dict(dtype=2, widths=(64,) * 7), 2),                             # fp64: up to five GEMMs
    (dict(widths=(128,) * 7), 2),                                     # 192 KB of weights
    (dict(widths=(128, 128, 128, 128, 64), flags=2 | (3 << 4)), 2),   # orientation N beyond three
    (dict(widths=(128, 96, 80, 64, 32)), 2),                          # a width off the granule
])
def test_chain_create_rejects(kw, status):
    st, h = _chain(**kw)
    assert st == status
    assert h.value is None


@pytest.mark.parametrize("kw,expect", [
    (dict(), dict(mfma="32x32x16", dims="128x128x128x128x64", remap="relabel")),
    (dict(dtype=1, widths=(64, 96, 128, 32, 128, 64, 128), flags=2 << 4),
     dict(mfma="32x32x16", dims="64x96x128x32x128x64x128", remap="permlane")),
    (dict(dtype=1, widths=(64, 96, 160, 32, 224, 64, 128)),
     dict(mfma="32x32x16", dims="64x96x160x32x224x64x128", remap="relabel")),
    (dict(widths=(64, 96, 64, 128, 32, 64, 96, 64)), dict(path="fused", dims="64x96x64x128x32x64x96x64", launches="1")),
    (dict(dtype=1, widths=(64, 64, 128, 64, 96, 32, 128, 64, 96)), dict(path="fused", mfma="32x32x16", launches="1")),
    # up to three GEMMs the chain call plans what b2b_gemm_create plans
    (dict(widths=(128, 128, 128)), dict(mfma="16x16x32", remap="relabel", mt="1")),
    (dict(widths=(128, 128, 128, 64)), dict(mfma="16x16x32", remap="relabel")),
    (dict(widths=(128, 128)), dict(mfma="16x16x32", dims="128x128")),   # one GEMM
    (dict(dtype=2, widths=(64, 48, 64, 32, 64)), dict(mfma="f64_16x16x4", dims="64x48x64x32x64")),
])
def test_chain_plan_selection(kw, expect):
    info = _chain_info(**kw)
    for k, v in expect.items():
        assert info[k] == v, (k, info)


def _typed(dtypes, widths, flags=0, batch=1, M=128):
    h = ctypes.c_void_p(123)
    n = len(widths) - 1
    ts = (ctypes.c_int32 * len(dtypes))(*dtypes) if dtypes is not None else None
    w = (ctypes.c_int64 * len(widths))(*widths)
    st = cf.lib().b2b_chain_create_typed(ctypes.byref(h), ts, batch, M, n, w, None, None, flags)
    info = None
    if st == 0:
        buf = ctypes.create_string_buffer(512)
        assert cf.lib().b2b_gemm_get_info(h, buf, 512) == 0
        info = dict(kv.split("=", 1) for kv in buf.value.decode().split())
        assert cf.lib().b2b_gemm_destroy(h) == 0
    else:
        assert h.value is None
    return st, info


@pytest.mark.parametrize("dtypes,widths,expect", [
    ((0, 1, 0), (128, 128, 128), dict(dtype="f16/bf16/f16", mfma="32x32x16", remap="relabel")),
    ((1, 0, 1), (256, 256, 64), dict(dtype="bf16/f16/bf16", mfma="32x32x16", lds_bytes="163840")),
    ((0, 1, 0, 1), (128, 96, 128, 64), dict(dtype="f16/bf16/f16/bf16", mfma="32x32x16", launches="1")),
    ((0, 0, 0, 1), (128, 128, 128, 64), dict(dtype="f16/f16/f16/bf16", path="fused")),
    # mixtures without a compiled mask: the types read at run time
    ((0, 1, 1, 0, 0), (128, 128, 128, 128, 64), dict(dtype="f16/bf16/bf16/f16/f16", mfma="32x32x16")),
    ((1, 0, 1, 0, 1, 0, 1), (64, 96, 128, 32, 128, 64, 128), dict(dtype="bf16/f16/bf16/f16/bf16/f16/bf16")),
    ((0, 1, 0, 1), (256, 64, 256, 64), dict(dtype="f16/bf16/f16/bf16", path="fused")),
    ((1, 0, 0, 1, 1, 0, 1, 0, 1), (64, 64, 128, 64, 96, 32, 128, 64, 96), dict(path="fused", launches="1")),
    ((0, 1, 0, 1, 1), (64, 32, 32, 32, 64), dict(dtype="f16/bf16/f16/bf16/bf16", path="fused")),
    # four and five typed GEMMs past 128 wide
    ((0, 1, 0, 1, 0), (256, 128, 128, 128, 64), dict(dtype="f16/bf16/f16/bf16/f16", path="fused",
                                                     mfma="32x32x16", launches="1")),
    ((1, 0, 1, 0, 1, 0), (256, 64, 192, 64, 128, 64), dict(dtype="bf16/f16/bf16/f16/bf16/f16", path="fused")),
    # one type throughout: the plan of b2b_chain_create
    ((1, 1, 1), (128, 128, 128), dict(dtype="bf16", mfma="16x16x32")),
    ((2, 2, 2), (64, 64, 64), dict(dtype="f64", mfma="f64_16x16x4")),
])
def test_typed_plan_selection(dtypes, widths, expect):
    st, info = _typed(dtypes, widths)
    assert st == 0
    for k, v in expect.items():
        assert info[k] == v, (k, info)


@pytest.mark.parametrize("dtypes,widths,flags,status", [
    (None, (128, 128, 128), 0, 1),
    ((0, 1, 0), (128, 128, 128), 2 << 4, 2),                      # lane-half swaps: not compiled typed
    ((0, 1, 0), (128, 128, 128), 2 | (3 << 4), 2),                # orientation N
    ((0, 2, 0), (64, 64, 64), 0, 2),                              # fp64 mixed with a 16-bit type
    ((0, 1, 0, 1, 0, 1, 0, 1), (128,) * 8, 0, 2),                 # 224 KB of weights
    ((0, 1, 0, 1, 0, 1, 0, 1, 0, 1), (64,) * 10, 0, 1),           # nine GEMMs
    ((0, 1, 0, 1, 0, 1, 0), (256, 64, 64, 64, 64, 64, 64), 0, 2),    # six or more typed GEMMs: widths up to 128
    ((0, 5, 0), (128, 128, 128), 0, 2),                           # unknown type
])
def test_typed_rejects(dtypes, widths, flags, status):
    st, _ = _typed(dtypes, widths, flags)
    assert st == status


@pytest.mark.parametrize("kw,expect", [
    (dict(dtype=3, widths=(128, 128, 128)), dict(dtype="tf32", mfma="bf16x3_32x32x16", waves="8",
                                                 lds_bytes=str(128 * 128 * 2 * 4 + 8 * 4096), widths="compiled")),
    (dict(dtype=3, widths=(128, 128, 128), flags=8), dict(mfma="bf16x4_32x32x16", widths="compiled")),
    (dict(dtype=3, widths=(128, 128, 128, 64)), dict(mfma="bf16x3_32x32x16", waves="8", rows_per_wg="256",
                                                     lds_bytes=str(160 * 1024), widths="compiled")),
    (dict(dtype=3, widths=(128, 128, 128, 64), flags=8), dict(mfma="bf16x4_32x32x16", widths="compiled")),
    # other widths: the same kernels reading the widths at run time
    (dict(dtype=3, widths=(128, 96, 128)), dict(waves="8", widths="runtime")),
    (dict(dtype=3, widths=(128, 128, 128, 32)), dict(rows_per_wg="256", widths="runtime")),
    (dict(dtype=3, widths=(96, 64)), dict(dims="96x64", launches="1", widths="runtime")),
    # the fixed-width 16-bit kernels have their widths compiled in
    (dict(dtype=0, widths=(128, 128, 128)), dict(widths="compiled")),
])
def test_tf32_plan_selection(kw, expect):
    info = _chain_info(**kw)
    for k, v in expect.items():
        assert info[k] == v, (k, info)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3, widths=(256, 128, 128)), 2),                   # widths up to 128
    (dict(dtype=3, widths=(128, 80, 128)), 2),                    # multiples of 32
    (dict(dtype=3, widths=(128,) * 5), 2),                        # fused: up to three GEMMs
    (dict(dtype=3, widths=(128, 128, 128), flags=2 << 4), 2),     # relabelled only
    (dict(dtype=0, widths=(128, 128, 128), flags=8), 1),          # the four-pass flag is for tf32
])
def test_tf32_rejects(kw, status):
    st, h = _chain(**kw)
    assert st == status and h.value is None


def test_typed_rejects_tf32_mix():
    st, _ = _typed((3, 0, 3), (128, 128, 128))
    assert st == 2
    st, info = _typed((3, 3, 3), (128, 128, 128))
    assert st == 0 and info["dtype"] == "tf32"


@pytest.mark.parametrize("dtypes,widths,expect", [
    # four waves: two workgroups a CU (48 KB of weights, 4 x 4 KB of D staging)
    ((0, 4, 0), (128, 128, 128), dict(dtype="f16/fp8/f16", mfma="32x32x16+f8_32x32x64", waves="4",
                                      lds_bytes=str(128 * 128 * 2 + 128 * 128 + 4 * 4096))),
    ((1, 4, 1), (256, 128, 256), dict(dtype="bf16/fp8/bf16", lds_bytes=str(256 * 128 * 2 + 128 * 256 + 8 * 4096))),
    ((0, 4, 1), (96, 64, 32), dict(dtype="f16/fp8/bf16", launches="1")),
])
def test_fp8_plan_selection(dtypes, widths, expect):
    st, info = _typed(dtypes, widths)
    assert st == 0
    for k, v in expect.items():
        assert info[k] == v, (k, info)


@pytest.mark.parametrize("dtypes,widths,flags,status", [
    ((0, 4, 0), (128, 96, 128), 0, 2),                 # N1 a multiple of 64
    ((0, 4, 0), (256, 256, 256), 0, 2),                # 192 KB of weights
    ((4, 0, 0), (128, 128, 128), 0, 2),                # fp8 is a later GEMM's type
    ((0, 0, 4), (128, 128, 128), 0, 2),                # not D's
    ((0, 4, 0, 0), (128, 128, 128, 64), 0, 2),         # two GEMMs
    ((0, 4, 0), (128, 128, 128), 2 << 4, 2),           # relabelled only
    ((0, 4, 0), (128, 128, 144), 0, 2),                # N2 a multiple of 32
])
def test_fp8_rejects(dtypes, widths, flags, status):
    st, _ = _typed(dtypes, widths, flags)
    assert st == status


def test_fp8_weights_leading_dimension_in_bytes():
    """B1 is one byte an element: its leading dimension needs 16 bytes, not 32."""
    h = ctypes.c_void_p(123)
    ts = (ctypes.c_int32 * 3)(0, 4, 0)
    w = (ctypes.c_int64 * 3)(128, 128, 32)
    ld = (ctypes.c_int64 * 4)(128, 128, 48, 32)
    assert cf.lib().b2b_chain_create_typed(ctypes.byref(h), ts, 1, 64, 2, w, ld, None, 0) == 0
    cf.lib().b2b_gemm_destroy(h)
    ld2 = (ctypes.c_int64 * 4)(128, 136, 48, 32)         # B0 (16-bit) needs multiples of 8 elements
    h2 = ctypes.c_void_p(123)
    assert cf.lib().b2b_chain_create_typed(ctypes.byref(h2), ts, 1, 64, 2, w, ld2, None, 0) == 0
    cf.lib().b2b_gemm_destroy(h2)
    ld3 = (ctypes.c_int64 * 4)(128, 128, 40, 32)         # 40 bytes: not a multiple of 16
    h3 = ctypes.c_void_p(123)
    assert cf.lib().b2b_chain_create_typed(ctypes.byref(h3), ts, 1, 64, 2, w, ld3, None, 0) == 1


def test_gemm_run_rejects_chain_plans():
    st, h = _chain()
    assert st == 0
    a = ctypes.c_void_p(0x1000)
    assert cf.lib().b2b_gemm_run(h, a, a, a, a, ctypes.c_void_p(0x2000), None) == 1
    ptrs = (ctypes.c_void_p * 4)(0x1000, 0x1000, None, 0x1000)
    assert cf.lib().b2b_chain_run(h, a, ptrs, ctypes.c_void_p(0x2000), None) == 1   # a NULL weight
    cf.lib().b2b_gemm_destroy(h)


def test_tune_rejects_bad_arguments():
    st, h = _create()
    assert st == 0
    L = cf.lib()
    As = (ctypes.c_void_p * 1)(0x1000)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    Ds = (ctypes.c_void_p * 1)(0x2000)
    assert L.b2b_gemm_tune(None, 1, As, ptrs, Ds, None, 5) == 1
    assert L.b2b_gemm_tune(h, 1, As, None, Ds, None, 5) == 1
    assert L.b2b_gemm_tune(h, 0, As, ptrs, Ds, None, 5) == 1
    assert L.b2b_gemm_tune(h, 1, As, ptrs, Ds, None, 0) == 1
    L.b2b_gemm_destroy(h)


def test_source_digest_ignores_comments_only():
    """The digest that ties stored profiler counters to the kernels reads code,
    not comments or layout."""
    from chip_fusion_amd import build
    a = "int f(int x) {\n  // doubled\n  return 2 * x; /* all */\n}\n"
    b = "int f(int x)\n{ return 2 * x;   // twice\n}"
    c = "int f(int x) { return 3 * x; }"
    assert build._code_only(a) == build._code_only(b) != build._code_only(c)
    assert len(build.source_digest()) == 16


def test_tile_count_beyond_32_bits_refused():
    """The kernels count row tiles in 32 bits: a plan whose batch x tiles would
    not fit is refused at creation (such inputs could not be allocated anyway)."""
    st, h = _create(batch=1 << 30, M=1 << 20)
    assert st == 1 and h.value is None
    st, h = _create(batch=1 << 10, M=1 << 20)           # 2^23 tiles of 128 rows: fine
    assert st == 0
    cf.lib().b2b_gemm_destroy(h)


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library the package raises ImportError at its first
    call; there is no fallback path."""
    pkg = tmp_path / "chip_fusion_amd"
    pkg.mkdir()
    src = os.path.join(ROOT, "chip_fusion_amd", "__init__.py")
    (pkg / "__init__.py").write_text(open(src).read())
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import chip_fusion_amd as cf\n"
            "for f in (cf.lib, lambda: cf.Plan('f16', 1, 128, 64, 64, 64)):\n"
            "    try:\n"
            "        f()\n"
            "    except ImportError as e:\n"
            "        print('ImportError', 'libb2b.so' in str(e))\n"
            "    else:\n"
            "        print('no error')\n") % str(tmp_path)
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.stdout.split() == ["ImportError", "True", "ImportError", "True"], r.stdout + r.stderr[-500:]


def test_leading_dimension_spans_below_2_31_accepted():
    """Just inside the 32-bit offsets: 32 rows of A at 2^24 - 8 elements, a
    64-row weight at 2^23 elements (2^30 bytes) and fp64 D at 2^22."""
    for kw in (dict(ld=[(1 << 24) - 8, 64, 64, 0, 64]), dict(ld=[64, 1 << 23, 64, 0, 64]),
               dict(dtype=2, ld=[64, 64, 64, 0, 1 << 22])):
        st, h = _create(**kw)
        assert st == 0, kw
        cf.lib().b2b_gemm_destroy(h)


def test_plan_log_on_request():
    """B2B_LOG=1 prints the chosen plan on stderr at creation; unset, nothing."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import chip_fusion_amd as cf\n"
            "cf.Plan('f16', 2, 100, 64, 64, 64).close()\n") % ROOT
    env = dict(os.environ, B2B_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-500:]
    line = [x for x in r.stderr.splitlines() if x.startswith("[b2b] plan:")]
    assert len(line) == 1 and "path=fused" in line[0] and "dims=64x64x64" in line[0] and "M=100" in line[0]
    env.pop("B2B_LOG")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    assert "[b2b]" not in r.stderr


def test_static_run_checks_before_touching_the_device():
    """b2b_chain_run_static plans and sizes its intermediates first: bad
    arguments and intermediates beyond the static workspace are refused
    before the device is touched."""
    L = cf.lib()
    p = ctypes.c_void_p(0x1000)
    ptrs = (ctypes.c_void_p * 3)(0x1000, 0x1000, 0x1000)

    def run(dtype, batch, M, widths):
        w = (ctypes.c_int64 * len(widths))(*widths)
        return L.b2b_chain_run_static(dtype, batch, M, len(widths) - 1, w, None, None, p, ptrs,
                                      ctypes.c_void_p(0x2000000), None)
    assert L.b2b_chain_run_static(0, 1, 64, 2, None, None, None, p, ptrs, ctypes.c_void_p(0x2000), None) == 1
    assert run(0, 0, 64, [64, 64, 64]) == 1                      # no batches
    # two GEMMs: one intermediate, the whole 32 MiB array
    assert run(0, 1, 131072, [64, 128, 64]) != 5                 # exactly 32 MiB fits
    assert run(0, 1, 131073, [64, 128, 64]) == 5                 # a row more does not
    # three GEMMs: two halves of the largest intermediate (16 MiB each)
    assert run(0, 1, 65536, [64, 128, 64, 64]) != 5
    assert run(0, 1, 65537, [64, 128, 64, 64]) == 5
    assert run(2, 8, 16384, [64, 64, 64]) == 5                   # fp64 workload 4: 64 MiB
    assert cf.STATIC_WORKSPACE_BYTES == 32 << 20


@pytest.mark.parametrize("kw,tail,mfma", [
    # widths off the granule: the tail kernels (32x32x16 for 16-bit, 16x16x4 for fp64)
    (dict(K=100, N1=72, N2=50), 1, "32x32x16"),
    (dict(dtype=1, K=100, N1=72, N2=50, N3=40), 1, "32x32x16"),
    (dict(K=1, N1=1, N2=1), 1, "32x32x16"),
    (dict(K=96, N1=80, N2=96), 1, "32x32x16"),
    (dict(dtype=2, K=10, N1=20, N2=36), 1, "f64_16x16x4"),
    (dict(dtype=2, K=10, N1=20, N2=36, N3=12), 1, "f64_16x16x4"),
    # whole granules, rows off 16-byte boundaries (dense or padded)
    (dict(ld=[68, 64, 64, 0, 64]), 1, "32x32x16"),
    (dict(dtype=2, ld=[65, 64, 64, 0, 64]), 1, "f64_16x16x4"),
    (dict(batch=2, bs=[128 * 64 + 4, 4096, 4096, 0, 128 * 64]), 1, "32x32x16"),
    # whole granules on 16-byte rows: the kernels without tails
    (dict(), 0, "16x16x32"),
    (dict(ld=[72, 64, 64, 0, 64]), 0, "16x16x32"),
])
def test_tail_plan_selection(kw, tail, mfma):
    """K and N tails, and rows at any element alignment, plan onto the tail
    kernels; whole granules on 16-byte rows keep the kernels without tails."""
    info = _info(**kw)
    assert info["tail"] == str(tail) and info["mfma"] == mfma and info["path"] == "fused", info


def test_tail_bounds():
    """Tails fuse within the padded bounds: 16-bit to 256 with all weights in
    LDS, fp64 to 64 for two or three GEMMs."""
    assert _create(K=250, N1=150, N2=130)[0] == 0
    assert _create(K=250, N1=250, N2=250)[0] == 2          # 2 x 256 x 256 x 2 bytes of weights
    assert _create(dtype=2, K=60, N1=60, N2=60)[0] == 0
    assert _create(dtype=2, K=60, N1=70, N2=60)[0] == 2    # 70 pads to 80 > 64


@pytest.mark.parametrize("kw,bound", [
    (dict(dtype=0, widths=(192, 160, 192)), "192"),        # instances bounded at 192 hold an A tile ahead
    (dict(dtype=0, widths=(96, 160, 64)), "192"),
    (dict(dtype=1, widths=(256, 128, 256)), "256"),
    (dict(dtype=0, widths=(192, 64, 192, 64, 192)), "192"),
    (dict(dtype=0, widths=(128, 128, 128)), "0"),          # the fixed-width kernel
    (dict(dtype=2, widths=(96, 96, 96)), "96"),            # fp64, two GEMMs up to 96
    (dict(dtype=2, widths=(96, 48, 112)), "128"),
    (dict(dtype=2, widths=(64, 64, 64, 64, 64)), "64"),
])
def test_width_bound_selection(kw, bound):
    """The planner takes the run-time-width instance with the smallest bound
    that holds every width (the fixed-width kernels report 0)."""
    assert _chain_info(**kw)["bound"] == bound
