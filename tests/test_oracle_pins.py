"""Pins of the plain CPU oracle against facts that do not come from the oracle itself:
IEEE 754 rounding as implemented by numpy / torch, exact integer arithmetic,
exact rational arithmetic with the standard dot-product error bound, closed
forms (identity and permutation weights) and invariants of the cascade
(batch and row independence, exact power-of-two scaling)."""
import threading
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


# ----------------------------------------------------------------------------
# 16-bit encoders / decoders
# ----------------------------------------------------------------------------
_CH = 1 << 24


class _Bufs(threading.local):
    def __init__(self):
        self.iota = np.arange(_CH, dtype=np.uint32)
        self.u = np.empty(_CH, np.uint32)
        self.ref16 = torch.empty(_CH, dtype=torch.float16)
        self.refb = np.empty(_CH, np.uint32)
        self.got = np.empty(_CH, np.uint16)
        self.ne = np.empty(_CH, bool)


_bufs = _Bufs()


def _mismatches(got, ref, x):
    """Indices where the encodings differ, ignoring NaN inputs that map to NaN."""
    np.not_equal(got, ref, out=_bufs.ne)
    idx = np.flatnonzero(_bufs.ne)
    return [int(i) for i in idx if not np.isnan(x[i])] if idx.size else []


def _f16_chunk(lo):
    b = _bufs
    np.add(b.iota, np.uint32(lo), out=b.u)
    x = b.u.view(np.float32)
    b.ref16.copy_(torch.from_numpy(x))                 # torch float32 -> float16, RNE
    oracle._load().oracle_encode_f16_array(oracle._ptr(x), oracle._ptr(b.got), _CH)
    bad = _mismatches(b.got, b.ref16.view(torch.int16).numpy().view(np.uint16), x)
    for i in bad:                                      # NaN must stay NaN
        assert not np.isnan(x[i])
    return len(bad)


def test_f16_encoder_exhaustive():
    """Every float32 bit pattern against torch's float32->float16 cast (RNE)."""
    torch.set_num_threads(1)
    with ThreadPoolExecutor(8) as ex:
        bad = sum(ex.map(_f16_chunk, range(0, 1 << 32, _CH)))
    assert bad == 0


def test_f16_encoder_matches_numpy():
    """A sample (all exponents, exact ties included) against numpy's cast too."""
    rng = np.random.default_rng(4)
    u = rng.integers(0, 1 << 32, 1 << 21, dtype=np.uint64).astype(np.uint32)
    u[: 1 << 19] = (u[: 1 << 19] & np.uint32(0xFFFFE000)) | np.uint32(0x1000)    # normal-range ties
    x = u.view(np.float32)
    fin = ~np.isnan(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.encode_f16(x)
    assert np.array_equal(got[fin], ref[fin])


def _bf16_ref(u, out):
    """Round-to-nearest-even on the low 16 bits, in plain numpy integer ops, as
    a second, independent bfloat16 reference (cross-checked against torch's
    cast on a sample below)."""
    np.right_shift(u, np.uint32(16), out=out)
    lowb = u & np.uint32(0xFFFF)
    up = (lowb > 0x8000) | ((lowb == 0x8000) & ((out & np.uint32(1)) == 1))
    out += up.astype(np.uint32)


def _bf16_chunk(lo):
    b = _bufs
    np.add(b.iota, np.uint32(lo), out=b.u)
    x = b.u.view(np.float32)
    _bf16_ref(b.u, b.refb)
    oracle._load().oracle_encode_bf16_array(oracle._ptr(x), oracle._ptr(b.got), _CH)
    bad = _mismatches(b.got, b.refb.astype(np.uint16), x)
    return len(bad)


def test_bf16_encoder_exhaustive():
    """Every float32 bit pattern against integer RNE on the encoding (non-NaN)."""
    with ThreadPoolExecutor(8) as ex:
        bad = sum(ex.map(_bf16_chunk, range(0, 1 << 32, _CH)))
    assert bad == 0


def test_bf16_encoder_matches_torch():
    """Sample of float32 patterns (all exponents, tie patterns included)
    against torch's float32 -> bfloat16 cast."""
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    u[: 1 << 20] = (u[: 1 << 20] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    x = u.view(np.float32)
    fin = ~np.isnan(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode_bf16(x)
    assert np.array_equal(got[fin], ref[fin])
    gotf = (got[~fin].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(gotf))


def test_decoders_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = oracle.decode_f16(h)
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[~fin]))
    gb = oracle.decode_bf16(h)
    assert np.array_equal(gb.view(np.uint32), h.astype(np.uint32) << 16)


def test_rounding_points():
    """Hand-checked binary16 cases: 1 + 3*2^-12 rounds up to 1 + 2^-10, the tie
    1 + 2^-11 rounds to the even 1, 65520 overflows, 2^-25 ties to 0 and
    3*2^-26 rounds to the smallest subnormal."""
    x = np.array([1 + 3 * 2.0 ** -12, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504, 65520,
                  2.0 ** -25, 3 * 2.0 ** -26, -2.0 ** -24], np.float32)
    want = [0x3C01, 0x3C00, 0x3C02, 0x7BFF, 0x7C00, 0x0000, 0x0001, 0x8001]
    assert [int(v) for v in oracle.encode_f16(x)] == want
    # bf16: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1); 1 + 3*2^-9 -> 1 + 2^-7
    xb = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -9, 1 + 3 * 2.0 ** -8], np.float32)
    assert [int(v) for v in oracle.encode_bf16(xb)] == [0x3F80, 0x3F81, 0x3F82]


# ----------------------------------------------------------------------------
# tf32 rounding
# ----------------------------------------------------------------------------
def _tf32_ref(x):
    """Nearest-even rounding of float32 values to 11 significant bits in
    float64 arithmetic (frexp / rint / ldexp), with the fixed 2^-136 quantum
    below 2^-126 and overflow to infinity past the largest tf32 value;
    independent of the oracle's integer rounding of the encoding."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    out[~fin] = x[~fin]
    xf = x[fin]
    m, e = np.frexp(xf)                             # xf = m 2^e, 0.5 <= |m| < 1
    q = np.where(np.abs(xf) >= 2.0 ** -126,
                 np.ldexp(np.rint(np.ldexp(m, 11)), e - 11),
                 np.ldexp(np.rint(np.ldexp(xf, 136)), -136))
    big = np.abs(q) > (2.0 - 2.0 ** -10) * 2.0 ** 127
    q[big] = np.copysign(np.inf, q[big])
    out[fin] = q
    return out


def test_tf32_rounding_against_float64_reference():
    """Every fraction pattern of the binade at 1 and of the subnormals, the
    lowest and highest 2^20 patterns of the smallest normal and the largest
    binade (the carry into the next binade and into infinity), 2^22 random
    encodings of either sign, and the specials."""
    full = [np.arange(1 << 23, dtype=np.uint32) | np.uint32(e << 23) for e in (127, 0)]
    low = np.arange(1 << 20, dtype=np.uint32)
    high = np.arange((1 << 23) - (1 << 20), 1 << 23, dtype=np.uint32)
    edges = [p | np.uint32(e << 23) for e in (1, 254) for p in (low, high)]
    rng = np.random.default_rng(5)
    rnd = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate(full + edges + [rnd])
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.round_tf32(x).astype(np.float64)
    want = _tf32_ref(x)
    bad = ~((got == want) | (np.isnan(got) & np.isnan(want)))
    assert not bad.any(), (x[bad][:5], got[bad][:5], want[bad][:5])
    sp = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0], np.float32)
    r = oracle.round_tf32(sp)
    assert r[0] == np.inf and r[1] == -np.inf and np.isnan(r[2])
    assert r[3] == 0.0 and not np.signbit(r[3]) and r[4] == 0.0 and np.signbit(r[4])


def test_tf32_rounding_points():
    """1 + 2^-11 is a tie between 1 and 1 + 2^-10 (-> 1, even); 1 + 3*2^-11
    a tie between 1 + 2^-10 and 1 + 2^-9 (-> 1 + 2^-9, even); the largest
    float32 rounds past the largest tf32 value (2 - 2^-10) 2^127 to infinity;
    the smallest subnormal is below half the tf32 quantum 2^-136."""
    x = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 + 2 ** -11 + 2 ** -20,
                  np.finfo(np.float32).max, 2.0 ** -149, 3 * 2.0 ** -137], np.float32)
    got = oracle.round_tf32(x).tolist()
    assert got == [1.0, 1 + 2 ** -9, 1 + 2 ** -10, np.inf, 0.0, 2.0 ** -135]


# ----------------------------------------------------------------------------
# fp8 E4M3
# ----------------------------------------------------------------------------
def test_fp8_decode_all_codes_match_torch():
    c = np.arange(256, dtype=np.uint8)
    got = oracle.decode_fp8(c).astype(np.float64)
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want)) and np.isnan(got).sum() == 2
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_fp8_encode_matches_torch():
    """Every float32 within +-480 on a fine grid (all ties of every binade
    included: the grid step 2^-12 divides every fp8 half-quantum), plus
    random float32 values across the whole range."""
    grid = np.arange(-480 * 4096, 480 * 4096 + 1, dtype=np.float64) / 4096.0
    rng = np.random.default_rng(9)
    rnd = (rng.standard_normal(1 << 20) * np.exp(rng.uniform(-20, 8, 1 << 20))).astype(np.float64)
    x = np.concatenate([grid, rnd, [2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -7 + 2.0 ** -10]]).astype(np.float32)
    got = oracle.encode_fp8(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = got != want
    assert not bad.any(), (x[bad][:5], got[bad][:5], want[bad][:5])


def test_fp8_encode_is_nearest_even():
    """Brute force: the code's value is a nearest finite fp8 value to x, and
    of two equally near ones the one with an even code."""
    vals = oracle.decode_fp8(np.arange(128, dtype=np.uint8)).astype(np.float64)[:127]   # +0 .. 448
    rng = np.random.default_rng(10)
    x = np.abs(rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000)))
    x = x[x < 464].astype(np.float32)
    codes = oracle.encode_fp8(x)
    d = np.abs(vals[None, :] - x.astype(np.float64)[:, None])
    best = d.min(axis=1)
    assert np.array_equal(d[np.arange(x.size), codes], best)
    ties = (d == best[:, None]).sum(axis=1) == 2
    assert np.all(codes[ties] % 2 == 0)


# ----------------------------------------------------------------------------
# One stage against exact rational arithmetic (tiny sizes)
# ----------------------------------------------------------------------------
def _exact(Xd, Bd):
    M, K = Xd.shape
    N = Bd.shape[1]
    return [[sum(Fraction(float(Xd[m, k])) * Fraction(float(Bd[k, n])) for k in range(K))
             for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f64", "tf32"])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_stage_within_dot_product_bound(dtype, seed):
    """|acc - exact| <= gamma_K * sum_k |x||b| (Higham, Accuracy and Stability of
    Numerical Algorithms, the recursive-summation dot-product bound), with the
    accumulator's unit roundoff: 2^-24 for float32, 2^-53 for float64.  For
    tf32 the exact products are those of the operands rounded to tf32."""
    M, K, N = 5, 13, 7
    X = synth.tensor(seed, 0, (M, K), dtype, "uniform")
    B = synth.tensor(seed, 1, (K, N), dtype, "uniform")
    acc = oracle.gemm_acc(dtype, X, B)
    Xd, Bd = oracle.decode(dtype, X).astype(np.float64), oracle.decode(dtype, B).astype(np.float64)
    if dtype == "tf32":
        Xd, Bd = _tf32_ref(Xd), _tf32_ref(Bd)
        assert not np.array_equal(Xd, oracle.decode(dtype, X))   # the rounding did something
    ex = _exact(Xd, Bd)
    u = 2.0 ** -53 if dtype == "f64" else 2.0 ** -24
    gamma = K * u / (1 - K * u)
    absdot = np.abs(Xd) @ np.abs(Bd)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(float(acc[m, n])) - ex[m][n])
            assert err <= Fraction(gamma) * Fraction(float(absdot[m, n])), (m, n)
    # and it is not accidentally exact-by-zero: the values are non-trivial
    assert np.abs(acc).max() > 0.1


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f64"])
def test_stage_transposed_operand_would_fail(dtype):
    """The stage multiplies X by B, not by B^T: on a non-symmetric B the exact
    product and its transpose-swapped variant differ, and the oracle matches
    the former exactly on small integers."""
    X = synth.to_dtype(np.array([[1.0, 2.0], [3.0, 4.0]]), dtype)
    B = synth.to_dtype(np.array([[5.0, 6.0], [7.0, 8.0]]), dtype)
    acc = oracle.gemm_acc(dtype, X, B)
    assert np.array_equal(acc.astype(np.float64), np.array([[19.0, 22.0], [43.0, 50.0]]))


# ----------------------------------------------------------------------------
# Whole cascade: exact integer arithmetic
# ----------------------------------------------------------------------------
def _np_round(dtype, x):
    """Library RNE of exact integers/float64 values into the dtype (numpy for
    binary16, torch for bfloat16), returned as float64 values."""
    x = np.asarray(x, np.float64)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    return x


def _exact_cascade(dtype, A, Bs):
    """Integer-valued cascade in int64, rounding each stage with the library
    cast; valid when every partial sum is an integer below 2^24 (exact in
    float32) -- the caller guarantees it."""
    x = oracle.decode(dtype, A).astype(np.float64)
    for B in Bs:
        b = oracle.decode(dtype, B).astype(np.float64)
        y = np.einsum("...mk,...kn->...mn", x.astype(np.int64), b.astype(np.int64)).astype(np.float64)
        assert np.abs(y).max() < 2 ** 24
        x = _np_round(dtype, y)
    return x


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_ternary_cascade_exact(cfg):
    """{-1,0,1} inputs at the workload's K and N: every partial sum is a small
    integer, so the result is independent of summation order and equals the
    int64 product rounded by the library cast (stage by stage)."""
    c = synth.WORKLOADS[cfg]
    A, Bs = synth.make_inputs(cfg, M=96, batch=min(2, c["batch"]), dist="ternary")
    D = oracle.cascade(c["dtype"], A, Bs)
    want = _exact_cascade(c["dtype"], A, Bs)
    got = oracle.decode(c["dtype"], D).astype(np.float64)
    assert np.array_equal(got, want)
    assert np.abs(want).max() > 8      # non-trivial magnitudes


@pytest.mark.parametrize("dtype,lims,dims", [("f16", [12, 12, 1], [64, 16, 16]),
                                             ("bf16", [6, 6, 6], [32, 32, 32]),
                                             ("f16", [3, 3, 3, 1], [32, 32, 8, 16]),
                                             ("bf16", [2, 2, 2, 2], [32, 32, 32, 16])])
def test_intermediate_rounding_exact(dtype, lims, dims):
    """Non-negative integers in [0, lim] (per operand) make an intermediate exceed the dtype's
    exact integer range (2048 for fp16, 256 for bf16), so it is really rounded;
    every partial sum stays an integer below 2^24, exact in float32.  The
    oracle must equal library-RNE of each exact stage."""
    rng = np.random.default_rng(7)
    A = synth.to_dtype(rng.integers(0, lims[0] + 1, (40, dims[0])), dtype)
    Bs = [synth.to_dtype(rng.integers(0, lims[s + 1] + 1, (dims[s], dims[s + 1])), dtype)
          for s in range(len(dims) - 1)]
    D = oracle.cascade(dtype, A, Bs)
    want = _exact_cascade(dtype, A, Bs)
    exact_limit = 2048 if dtype == "f16" else 256
    x = oracle.decode(dtype, A).astype(np.int64)
    rounded = False
    for B in Bs[:-1]:
        x = x @ oracle.decode(dtype, B).astype(np.int64)
        rounded |= bool(np.abs(x).max() > exact_limit)
        x = _np_round(dtype, x).astype(np.int64)
    assert rounded      # an intermediate was really rounded
    assert np.all(np.isfinite(want))
    assert np.array_equal(oracle.decode(dtype, D).astype(np.float64), want)


@pytest.mark.parametrize("types,lims,dims", [(("f16", "bf16", "f16"), [6, 6, 6], [32, 32, 32]),
                                             (("bf16", "f16", "bf16"), [12, 12, 1], [64, 16, 16]),
                                             (("f16", "bf16", "f16", "bf16"), [3, 3, 3, 2], [32, 32, 16, 16]),
                                             (("bf16", "bf16", "f16", "f16"), [3, 3, 2, 1], [32, 32, 16, 4])])
def test_typed_intermediate_rounding_exact(types, lims, dims):
    """A type per stage: integer inputs whose intermediates exceed the exact
    integer range of the type they are rounded into (256 for bf16, 2048 for
    fp16).  The oracle must equal the exact int64 stage rounded by the library
    cast of that stage's type (numpy for binary16, torch for bfloat16), and
    must differ from the same inputs read as one uniform type."""
    rng = np.random.default_rng(17)
    A = synth.to_dtype(rng.integers(0, lims[0] + 1, (40, dims[0])), types[0])
    Bs = [synth.to_dtype(rng.integers(0, lims[s + 1] + 1, (dims[s], dims[s + 1])), types[s])
          for s in range(len(dims) - 1)]
    D = oracle.cascade(list(types), A, Bs)
    x = oracle.decode(types[0], A).astype(np.int64)
    rounded = False
    for s, B in enumerate(Bs):
        y = x @ oracle.decode(types[s], B).astype(np.int64)
        assert np.abs(y).max() < 2 ** 24
        limit = 2048 if types[s + 1] == "f16" else 256
        rounded |= bool(s + 1 < len(Bs) and np.abs(y).max() > limit)
        x = _np_round(types[s + 1], y).astype(np.int64)
    assert rounded
    got = oracle.decode(types[-1], D).astype(np.float64)
    assert np.array_equal(got, x.astype(np.float64))


@pytest.mark.parametrize("types", [("f16", "fp8", "f16"), ("bf16", "fp8", "bf16")])
def test_fp8_stage_integers_exact(types):
    """A 16-bit first GEMM feeding an fp8 second: small non-negative integers
    make intermediates up to ~200, which fp8 holds only to 4 significant bits,
    so they are really rounded (by the library cast, torch float8_e4m3fn); the
    fp8 weights are ternary; every partial sum is an exact float32 integer."""
    rng = np.random.default_rng(31)
    A = synth.to_dtype(rng.integers(0, 4, (60, 64)), types[0])
    B0 = synth.to_dtype(rng.integers(0, 2, (64, 64)), types[0])
    B1 = synth.to_dtype(rng.integers(-1, 2, (64, 32)), "fp8")
    D = oracle.cascade(list(types), A, [B0, B1])
    x = oracle.decode(types[0], A).astype(np.int64) @ oracle.decode(types[0], B0).astype(np.int64)
    assert x.max() > 64                                   # past 16: spacing 2 and more
    xr = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert not np.array_equal(xr, x)
    y = xr.astype(np.int64) @ oracle.decode("fp8", B1).astype(np.int64)
    assert np.array_equal(oracle.decode(types[2], D).astype(np.float64), _np_round(types[2], y))


def test_typed_rounding_points():
    """fp16 values through identity weights into a bf16 intermediate and back
    to fp16: 1 + 2^-8 is a tie between bf16 neighbours 1 and 1 + 2^-7 (-> 1,
    even), 1 + 3*2^-9 goes up to 1 + 2^-7, 1.5 and 2^-14 are exact in both;
    the bf16 results are exact in fp16 again.  With the intermediate in fp16
    instead, every value comes through unchanged."""
    vals = np.array([[1 + 2 ** -8, 1 + 3 * 2 ** -9, 1.5, 2.0 ** -14]], np.float32)
    A = oracle.encode("f16", vals)
    I16 = oracle.encode("f16", np.eye(4, dtype=np.float32))
    Ib = oracle.encode("bf16", np.eye(4, dtype=np.float32))
    D = oracle.cascade(["f16", "bf16", "f16"], A, [I16, Ib])
    assert oracle.decode("f16", D).tolist() == [[1.0, 1 + 2 ** -7, 1.5, 2.0 ** -14]]
    D2 = oracle.cascade(["f16", "f16", "bf16"], A, [I16, I16])
    assert oracle.decode("bf16", D2).tolist() == [[1.0, 1 + 2 ** -7, 1.5, 2.0 ** -14]]
    assert np.array_equal(oracle.cascade(["f16", "f16", "f16"], A, [I16, I16]), A)


@pytest.mark.parametrize("lims,dims", [([2047, 3, 1], [16, 16, 16]), ([40, 40, 2, 1], [32, 32, 16, 8])])
def test_tf32_cascade_integers_exact(lims, dims):
    """Integer operands exact in tf32 (below 2^11) whose stage results grow
    past 2^11, so they are rounded to tf32 when the next GEMM takes them;
    every partial sum is an integer below 2^24, exact in float32.  The oracle
    must equal the exact int64 stages with the float64 tf32 reference rounding
    each intermediate, and D unrounded."""
    rng = np.random.default_rng(29)
    A = rng.integers(-lims[0], lims[0] + 1, (50, dims[0])).astype(np.float32)
    Bs = [rng.integers(-lims[s + 1], lims[s + 1] + 1, (dims[s], dims[s + 1])).astype(np.float32)
          for s in range(len(dims) - 1)]
    D = oracle.cascade("tf32", A, Bs)
    x = A.astype(np.int64)
    rounded = False
    for s, B in enumerate(Bs):
        y = x @ B.astype(np.int64)
        assert np.abs(y).max() < 2 ** 24
        if s + 1 < len(Bs):
            r = _tf32_ref(y.astype(np.float64))
            rounded |= bool((r != y).any())
            x = r.astype(np.int64)
        else:
            x = y
    assert rounded
    assert D.dtype == np.float32 and np.array_equal(D.astype(np.float64), x.astype(np.float64))


def test_tf32_identity_and_permutation():
    """Identity weights give tf32(A) (the first GEMM rounds A, the second
    takes an exact tf32 value); permutation weights permute those columns."""
    n = 32
    A = synth.tensor(13, 0, (2, 40, n), "tf32", "normal")
    eye = np.broadcast_to(np.eye(n, dtype=np.float32), (2, n, n)).copy()
    D = oracle.cascade("tf32", A, [eye, eye])
    want = _tf32_ref(A).astype(np.float32)
    assert np.array_equal(D, want) and not np.array_equal(D, A)
    p = np.random.default_rng(4).permutation(n)
    P = np.zeros((n, n), np.float32); P[p, np.arange(n)] = 1.0
    D2 = oracle.cascade("tf32", A[0], [P, eye[0]])
    assert np.array_equal(D2, want[0][:, p])


# ----------------------------------------------------------------------------
# Closed forms and invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,nst", [("f16", 2), ("bf16", 2), ("f64", 2), ("f16", 3)])
def test_identity_weights(dtype, nst):
    n = 32
    A = synth.tensor(11, 0, (3, 50, n), dtype, "uniform")
    eye = synth.to_dtype(np.broadcast_to(np.eye(n), (3, n, n)), dtype)
    D = oracle.cascade(dtype, A, [eye] * nst)
    assert np.array_equal(D, A)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f64"])
def test_permutation_weights(dtype):
    n = 48
    rng = np.random.default_rng(3)
    p, q = rng.permutation(n), rng.permutation(n)
    P = np.zeros((n, n)); P[p, np.arange(n)] = 1.0    # (A P)[:, j] = A[:, p[j]]
    Q = np.zeros((n, n)); Q[q, np.arange(n)] = 1.0
    A = synth.tensor(12, 0, (70, n), dtype, "normal")
    D = oracle.cascade(dtype, A, [synth.to_dtype(P, dtype), synth.to_dtype(Q, dtype)])
    assert np.array_equal(D, A[:, p][:, q])


def test_power_of_two_scaling():
    dtype = "f16"
    A, Bs = synth.make_inputs(1, M=64)
    D = oracle.decode(dtype, oracle.cascade(dtype, A, Bs))
    A2 = synth.to_dtype(oracle.decode(dtype, A).astype(np.float64) * 2.0, dtype)
    D2 = oracle.decode(dtype, oracle.cascade(dtype, A2, Bs))
    x1 = oracle.decode(dtype, oracle.cascade(dtype, A, Bs[:1]))
    nz = np.abs(x1[x1 != 0])
    assert nz.min() >= 2.0 ** -13 and np.abs(D[D != 0]).min() >= 2.0 ** -13   # no subnormal rounding
    assert np.array_equal(D2, 2.0 * D)


def test_batch_and_row_independence():
    A, Bs = synth.make_inputs(5, M=40, batch=3)
    D = oracle.cascade("f16", A, Bs)
    for b in range(3):
        Db = oracle.cascade("f16", A[b], [x[b] for x in Bs])
        assert np.array_equal(D[b], Db)
    rows = np.array([0, 119, 41, 80, 5])
    Dr = oracle.cascade("f16", A, Bs, rows=rows)
    flat = D.reshape(-1, D.shape[-1])
    assert np.array_equal(Dr, flat[rows])
    assert np.array_equal(oracle.cascade("f16", A, Bs, nthreads=1), D)


def test_f64_cascade_against_exact_rationals():
    """Tiny fp64 cascade: within the dot-product bound of the exact rational
    cascade (the fp64 oracle does not round between stages)."""
    A = synth.tensor(21, 0, (4, 6), "f64", "uniform")
    B0 = synth.tensor(21, 1, (6, 5), "f64", "uniform")
    B1 = synth.tensor(21, 2, (5, 3), "f64", "uniform")
    D = oracle.cascade("f64", A, [B0, B1])
    x1 = _exact(A, B0)
    ex = [[sum(x1[m][k] * Fraction(float(B1[k, n])) for k in range(5)) for n in range(3)]
          for m in range(4)]
    mag = (np.abs(A) @ np.abs(B0)) @ np.abs(B1)
    for m in range(4):
        for n in range(3):
            assert abs(Fraction(float(D[m, n])) - ex[m][n]) <= Fraction(1e-14) * Fraction(float(mag[m, n]))
