"""Seeded synthetic inputs for the cascaded-GEMM workloads.

Shared by the tests, the benchmark and the smoke check; holds none of the
cascade's arithmetic (no products, no accumulation, no rounding of results).

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) used as a counter-based stream: output i of a
stream with seed s is mix(s + (i + 1) * 0x9E3779B97F4A7C15), with the published
mix constants.  Each tensor has its own stream, seed ^ (tensor_id << 32) with
A = 0, B0 = 1, B1 = 2, B2 = 3; elements are drawn batch-major, then row-major.

  uniform(0,1):   ((x >> 11) + 0.5) * 2^-53          (never 0 or 1)
  uniform(-1,1):  2u - 1
  normal(0,1):    Box-Muller on consecutive pairs (u1, u2): cos branch first,
                  then sin
  ternary:        floor(3u) - 1, i.e. {-1, 0, 1}

Values are drawn in float64 and rounded to nearest-even into the input type
(fp16 / bf16); fp64 inputs are kept as drawn.  16-bit inputs are returned as
their uint16 encodings, fp64 as float64.
"""
import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# The five workloads: (dtype, batch, M, [K, N1, N2(, N3)], distribution, scale, base seed)
WORKLOADS = {
    1: dict(name="fp16 b1 128x64 . 64x64 . 64x64", dtype="f16", batch=1, M=128,
            dims=[64, 64, 64], dist="uniform", scale=1.0, seed=0x5EED0001),
    2: dict(name="fp16 b64 4096x128 . 128x128 . 128x128", dtype="f16", batch=64, M=4096,
            dims=[128, 128, 128], dist="normal", scale=1 / math.sqrt(128), seed=0x5EED0002),
    3: dict(name="bf16 b1 65536x256 . 256x256 . 256x256", dtype="bf16", batch=1, M=65536,
            dims=[256, 256, 256], dist="normal", scale=1 / math.sqrt(256), seed=0x5EED0003),
    4: dict(name="fp64 b8 16384x64 . 64x64 . 64x64", dtype="f64", batch=8, M=16384,
            dims=[64, 64, 64], dist="uniform", scale=1.0, seed=0x5EED0004),
    5: dict(name="fp16 b16 32768x128 . 128x128 . 128x128 . 128x64", dtype="f16", batch=16,
            M=32768, dims=[128, 128, 128, 64], dist="normal", scale=1 / math.sqrt(128),
            seed=0x5EED0005),
}


_CHUNK = 1 << 20


def _pool():
    import concurrent.futures
    import os
    global _POOL
    if "_POOL" not in globals():
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _chunked(n, fn, out):
    """Fills out[a:b] = fn(a, b) over chunks, in threads (numpy drops the GIL)."""
    spans = [(a, min(n, a + _CHUNK)) for a in range(0, n, _CHUNK)]
    list(_pool().map(lambda ab: out.__setitem__(slice(*ab), fn(*ab)), spans))
    return out


def _mix(seed, a, b):
    with np.errstate(over="ignore"):
        z = np.arange(a + 1, b + 1, dtype=np.uint64)
        z *= GAMMA
        z += np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
        return z


def splitmix64(seed, n):
    """Outputs 0 .. n-1 of the SplitMix64 stream with this seed."""
    return _chunked(n, lambda a, b: _mix(seed, a, b), np.empty(n, np.uint64))


def _u01(seed, a, b):
    x = _mix(seed, a, b)
    x >>= np.uint64(11)
    u = x.astype(np.float64)
    u += 0.5
    u *= 2.0 ** -53
    return u


def uniform01(seed, n):
    return _chunked(n, lambda a, b: _u01(seed, a, b), np.empty(n, np.float64))


def _normal_chunk(seed, a, b):
    # a, b are pair indices: pair p uses stream outputs 2p, 2p+1
    u = _u01(seed, 2 * a, 2 * b)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * np.pi * u2
    out = np.empty(2 * (b - a))
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out


def draw(seed, n, dist, scale=1.0):
    if dist == "uniform":
        v = uniform01(seed, n)
        v *= 2.0
        v -= 1.0
        if scale != 1.0:
            v *= scale
        return v
    if dist == "normal":
        m = (n + 1) // 2
        out = np.empty(2 * m)
        spans = [(a, min(m, a + _CHUNK)) for a in range(0, m, _CHUNK)]
        list(_pool().map(lambda ab: out.__setitem__(slice(2 * ab[0], 2 * ab[1]),
                                                    _normal_chunk(seed, *ab)), spans))
        out = out[:n]
        out *= scale
        return out
    if dist == "ternary":
        return np.floor(3.0 * uniform01(seed, n)) - 1.0
    raise ValueError(dist)


def _rne_bf16_bits(x):
    """float64 -> nearest-even bfloat16 encoding (8 significand bits)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # exact in float32 for the bf16 range
    bits = q.astype(np.float32).view(np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16)


def _rne_fp8_codes(x):
    """float64 values within +-448 -> nearest-even fp8 E4M3 codes (4
    significant bits; fixed quantum 2^-9 below 2^-6)."""
    x = np.asarray(x, np.float64)
    if np.any(np.abs(x) > 448):
        raise ValueError("fp8 inputs must lie within +-448")
    a = np.abs(x)
    m, e = np.frexp(a)                                   # a = m 2^e, leading bit 2^(e-1)
    lead = np.where(a > 0, e - 1, -6)
    qexp = np.maximum(lead, -6) - 3
    q = np.ldexp(np.rint(np.ldexp(a, -qexp)), qexp)      # rounded magnitude
    m2, e2 = np.frexp(q)
    normal = q >= 2.0 ** -6
    ef = np.where(normal, e2 - 1 + 7, 0)
    fr = np.where(normal, np.rint((m2 * 2 - 1) * 8), np.rint(q / 2.0 ** -9))
    code = (ef.astype(np.int64) << 3) + fr.astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def to_dtype(x, dtype):
    x = np.asarray(x, np.float64)
    shape = x.shape
    x = x.reshape(-1)
    if dtype == "f16":
        return _chunked(x.size, lambda a, b: x[a:b].astype(np.float16).view(np.uint16),
                        np.empty(x.size, np.uint16)).reshape(shape)
    if dtype == "bf16":
        return _chunked(x.size, lambda a, b: _rne_bf16_bits(x[a:b]),
                        np.empty(x.size, np.uint16)).reshape(shape)
    if dtype == "f64":
        return x.reshape(shape)
    if dtype == "fp8":                  # E4M3 codes, nearest-even (inputs stay within +-448)
        return _chunked(x.size, lambda a, b: _rne_fp8_codes(x[a:b]),
                        np.empty(x.size, np.uint8)).reshape(shape)
    if dtype == "tf32":                 # float32 storage; the cascade rounds operands to tf32 itself
        return _chunked(x.size, lambda a, b: x[a:b].astype(np.float32),
                        np.empty(x.size, np.float32)).reshape(shape)
    raise ValueError(dtype)


def tensor(seed, tensor_id, shape, dtype, dist, scale=1.0):
    n = int(np.prod(shape))
    v = draw(seed ^ (tensor_id << 32), n, dist, scale)
    return to_dtype(v, dtype).reshape(shape)


def make_inputs(cfg, M=None, batch=None, dist=None, seed=None, types=None):
    """Inputs of a workload: returns (A, [B0, B1, (B2)]).

    cfg: a WORKLOADS key or dict.  M / batch / dist / seed override the
    workload's values (smaller sizes for the parity tests, 'ternary' for the
    exactness variants).  types: one 16-bit type per GEMM (A and B_0 in
    types[0], B_s in types[s]) instead of the workload's single type.
    """
    c = dict(WORKLOADS[cfg]) if isinstance(cfg, int) else dict(cfg)
    M = c["M"] if M is None else M
    batch = c["batch"] if batch is None else batch
    dist = c["dist"] if dist is None else dist
    seed = c["seed"] if seed is None else seed
    scale = c["scale"] if dist != "ternary" else 1.0
    dims = c["dims"]
    ty = types if types is not None else [c["dtype"]] * len(dims)
    A = tensor(seed, 0, (batch, M, dims[0]), ty[0], dist, scale)
    Bs = [tensor(seed, 1 + s, (batch, dims[s], dims[s + 1]), ty[s], dist, scale)
          for s in range(len(dims) - 1)]
    return A, Bs
