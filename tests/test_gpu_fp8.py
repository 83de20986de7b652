"""An fp8 second GEMM (b2b_chain_create_typed with {t0, FP8_E4M3, tD}): the
first GEMM in fp16/bf16 on the 32x32x16 instruction, its result rounded to
E4M3 on chip and multiplied by the fp8 B1 on v_mfma_scale_f32_32x32x64_f8f6f4.

Probes first: the kernels' conversion (v_cvt_pk_fp8_f32) against the oracle's
E4M3 encoder (bit for bit, in range), and the fp8 instruction's pairing of A
and B slots (the relabelled K order needs only that both operands pair lane
half h, slot u with the same k) on exact small integers.  Then parity with
the oracle's typed cascade within the fp16/bf16 tolerances, and bit-exact
integer cases whose intermediates fp8 really rounds."""
import math

import numpy as np
import pytest
import torch

import chip_fusion_amd as cf
import oracle
import synth
from gpu_common import assert_close, check_fp8_stage, nan_output

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(f"\n[case] {msg}", flush=True)


def test_fp8_conversion_matches_oracle():
    _flush("fp8 conversion probe")
    rng = np.random.default_rng(3)
    special = [0.0, -0.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -9, 2.0 ** -6,
               448.0, 460.0, 464.0, -464.0, 15.5, 17.0, 0.3, -0.3, 240.0, 248.0]
    x = np.concatenate([special, rng.standard_normal(256 - len(special)) * np.exp(rng.uniform(-8, 5, 256 - len(special)))])
    x = np.clip(x, -464, 464).astype(np.float32)
    x[-4:] = [-2.0 ** -11, -3 * 2.0 ** -12, -1e-6, -0.0]      # negative values that round to zero
    got = cf.fp8_convert_probe(torch.from_numpy(x).cuda()).cpu().numpy()
    want = oracle.encode_fp8(x)
    # a negative value that rounds to zero: the oracle keeps the sign (-0,
    # 0x80), the hardware gives +0 (0x00); the same number either way
    zero = (want & 0x7F) == 0
    assert np.all(got[zero] & 0x7F == 0) and np.all(got[zero & (x > 0)] == 0)
    bad = (got != want) & ~zero
    assert not bad.any(), (x[bad][:8], got[bad][:8], want[bad][:8])


def test_fp8_instruction_pairs_slots():
    _flush("fp8 instruction probe")
    rng = np.random.default_rng(4)
    av = rng.integers(-3, 4, (64, 32)).astype(np.float64)
    bv = rng.integers(-3, 4, (64, 32)).astype(np.float64)
    a = torch.from_numpy(synth.to_dtype(av, "fp8")).cuda()
    b = torch.from_numpy(synth.to_dtype(bv, "fp8")).cuda()
    c = cf.mfma_probe("fp8_32x32x64", a, b).cpu().numpy().astype(np.float64)
    # C[i][j] = sum over halves h and slots u of a[i + 32h][u] b[j + 32h][u];
    # lane l holds column j = l%32, rows 8(v/4) + 4(l/32) + v%4
    C = av[:32] @ bv[:32].T + av[32:] @ bv[32:].T
    want = np.empty((64, 16))
    for l in range(64):
        for v in range(16):
            want[l, v] = C[8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32]
    assert np.array_equal(c, want)


def _inputs(types, batch, M, widths, seed=0x5EED0600):
    A = synth.tensor(seed, 0, (batch, M, widths[0]), types[0], "normal", 1.0)
    B0 = synth.tensor(seed, 1, (batch, widths[0], widths[1]), types[0], "normal", 1.0 / math.sqrt(widths[0]))
    B1 = synth.tensor(seed, 2, (batch, widths[1], widths[2]), "fp8", "normal", 1.0 / math.sqrt(widths[1]))
    return A, [B0, B1]


def _run(types, A, Bs, ld=None, bs=None):
    batch, M, K = A.shape
    widths = [K, Bs[0].shape[2], Bs[1].shape[2]]
    Ad, B0d, B1d = cf.to_device(A, types[0]), cf.to_device(Bs[0], types[0]), cf.to_device(Bs[1], "fp8")
    D = nan_output(types[2], batch, M, widths[2])
    p = cf.Chain(list(types), batch, M, widths)
    info = p.info()
    p.run(Ad, B0d, B1d, D=D)
    torch.cuda.synchronize()
    p.close()
    return cf.to_host(D), info


CASES = [
    (("f16", "fp8", "f16"), 2, 300, (128, 128, 128)),
    (("bf16", "fp8", "bf16"), 1, 513, (256, 128, 256)),
    (("f16", "fp8", "bf16"), 3, 260, (96, 64, 32)),
    (("bf16", "fp8", "f16"), 1, 700, (64, 128, 96)),
    (("f16", "fp8", "f16"), 2, 129, (256, 256, 64)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fp8_second_gemm_parity(case):
    types, batch, M, widths = CASES[case]
    _flush(f"fp8 stage {types} batch={batch} M={M} widths={widths}")
    A, Bs = _inputs(types, batch, M, widths)
    got, info = _run(types, A, Bs)
    assert "mfma=32x32x16+f8_32x32x64" in info and "dtype=" + "/".join(types) in info, info
    flips = check_fp8_stage(types, A, Bs[0], Bs[1], got, lambda a, bs: _run(types, a, bs)[0],
                            f"fp8 {types} {widths}")
    print(f"intermediates rounded the other way at a tie: {flips}", flush=True)


@pytest.mark.parametrize("types", [("f16", "fp8", "f16"), ("bf16", "fp8", "bf16")])
def test_fp8_second_gemm_integers_exact(types):
    """Intermediates up to ~100 (fp8 keeps 4 significant bits: spacing 8
    above 64), ternary fp8 weights, exact float32 partial sums."""
    _flush(f"fp8 stage exact {types}")
    rng = np.random.default_rng(33)
    A = synth.to_dtype(rng.integers(0, 4, (2, 300, 64)), types[0])
    B0 = synth.to_dtype(rng.integers(0, 2, (2, 64, 128)), types[0])
    B1 = synth.to_dtype(rng.integers(-1, 2, (2, 128, 64)), "fp8")
    ref = oracle.cascade(list(types), A, [B0, B1])
    x = np.einsum("bmk,bkn->bmn", oracle.decode(types[0], A).astype(np.int64),
                  oracle.decode(types[0], B0).astype(np.int64))
    assert x.max() > 64
    got, _ = _run(types, A, [B0, B1])
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"


def test_fp8_padded_and_broadcast():
    types, M, batch, widths = ("f16", "fp8", "f16"), 300, 3, (64, 128, 96)
    _flush(f"fp8 strided widths={widths}")
    A, Bs = _inputs(types, batch, M, widths)
    Bs = [Bs[0], Bs[1].copy()]
    Bs[1][:] = Bs[1][0]                       # B1 broadcast to every batch
    lda, ldb0, ldb1, ldd = widths[0] + 8, widths[1] + 16, widths[2] + 32, widths[2] + 8
    sA, sB0, sD = M * lda + 8, widths[0] * ldb0 + 24, M * ldd + 16

    def padded(x, b, rows, cols, ld, stride, dt, fill):
        buf = torch.full(((b - 1) * stride + rows * ld + 64,), fill, dtype=dt, device="cuda")
        buf.as_strided((b, rows, cols), (stride, ld, 1)).copy_(x)
        return buf

    Ad = padded(cf.to_device(A, "f16"), batch, M, widths[0], lda, sA, torch.float16, float("nan"))
    B0d = padded(cf.to_device(Bs[0], "f16"), batch, widths[0], widths[1], ldb0, sB0, torch.float16, float("nan"))
    B1d = padded(cf.to_device(Bs[1][:1], "fp8"), 1, widths[1], widths[2], ldb1, 0, torch.uint8, 0x7F)
    Dd = torch.full(((batch - 1) * sD + M * ldd + 64,), float("nan"), dtype=torch.float16, device="cuda")
    p = cf.Chain(list(types), batch, M, list(widths), ld=[lda, ldb0, ldb1, ldd], batch_stride=[sA, sB0, 0, sD])
    p.run(Ad, B0d, B1d, D=Dd)
    torch.cuda.synchronize()
    p.close()
    view = Dd.as_strided((batch, M, widths[2]), (sD, ldd, 1))
    assert_close("f16", cf.to_host(view.contiguous()), oracle.cascade(list(types), A, Bs), "fp8 strided")
    mask = torch.ones_like(Dd, dtype=torch.bool)
    mask.as_strided((batch, M, widths[2]), (sD, ldd, 1)).fill_(False)
    assert torch.isnan(Dd[mask]).all().item(), "writes outside the output windows"


@pytest.mark.parametrize("types,widths", [(("f16", "fp8", "f16"), (128, 128, 128)),
                                          (("bf16", "fp8", "bf16"), (256, 256, 64)),
                                          (("f16", "fp8", "bf16"), (96, 64, 32))])
def test_fp8_unfused_matches_fused_bitwise(types, widths):
    """The unfused comparison (the first GEMM writes its result as E4M3 bytes,
    a second kernel multiplies them on the fp8 instruction) reads the
    intermediate in the fused kernel's slot order and sums in the same order:
    D agrees bit for bit, and with the oracle within the tolerance."""
    _flush(f"fp8 unfused {types} {widths}")
    batch, M = 2, 300
    A, Bs = _inputs(types, batch, M, widths)
    fused, _ = _run(types, A, Bs)
    Ad, B0d, B1d = cf.to_device(A, types[0]), cf.to_device(Bs[0], types[0]), cf.to_device(Bs[1], "fp8")
    D = nan_output(types[2], batch, M, widths[2])
    p = cf.Chain(list(types), batch, M, list(widths), unfused=True)
    info = p.info()
    p.run(Ad, B0d, B1d, D=D)
    torch.cuda.synchronize()
    p.close()
    assert "path=unfused" in info and "launches=2" in info, info
    unf = cf.to_host(D)
    assert np.array_equal(unf, fused), f"{int((unf != fused).sum())} elements differ"
    assert_close(types[2], unf, oracle.cascade(list(types), A, Bs), f"fp8 unfused {types}")
