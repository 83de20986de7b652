"""Plain CPU oracle of the fused cascaded GEMM and of its register rearrangement.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package; the product library never imports, links or
calls it, and it imports nothing from the product.

* ``cascade`` / ``gemm_acc`` / the 16-bit encoders wrap ``b2b_oracle.c`` (plain
  C, built with gcc, no fast-math) -- the value of the cascade of GEMMs the
  pages fuse (page 1, detailed description: the cascaded-GEMM definition and the
  three-operator cascade).
* ``remap`` holds the rearrangement oracle: register layouts, the relation
  between the first operator's result and the second operator's input, the
  coordination matrix and its replay (page 1, the relation between the first
  and second rearrangement group matrices, Figs. 2a/2b/3, and the coordination
  matrix of Fig. 4 with its encoding into f, g, h).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16, F64, TF32, FP8 = 0, 1, 2, 3, 4
_NAMES = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16,
          "f64": F64, "fp64": F64, "float64": F64, "tf32": TF32, "fp8": FP8, "e4m3": FP8}

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.library_path()
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_gemm_acc.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp]
        lib.oracle_gemm_acc.restype = ctypes.c_int
        lib.oracle_cascade.argtypes = [ctypes.c_int, ctypes.c_int, vp, i64, i64, vp, vp, vp, i64,
                                       vp, ctypes.c_int]
        lib.oracle_cascade.restype = ctypes.c_int
        lib.oracle_cascade_typed.argtypes = [vp, ctypes.c_int, vp, i64, i64, vp, vp, vp, i64, vp, ctypes.c_int]
        lib.oracle_cascade_typed.restype = ctypes.c_int
        for n in ("oracle_encode_f16_array", "oracle_encode_bf16_array",
                  "oracle_decode_f16_array", "oracle_decode_bf16_array", "oracle_round_tf32_array",
                  "oracle_encode_fp8_array", "oracle_decode_fp8_array"):
            getattr(lib, n).argtypes = [vp, vp, i64]
            getattr(lib, n).restype = None
        _lib = lib
    return _lib


def dtype_code(dtype):
    if isinstance(dtype, int):
        return dtype
    return _NAMES[str(dtype)]


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(dt, x):
    """16-bit inputs travel as their uint16 encodings, fp64 as float64, tf32
    as the float32 values it rounds."""
    if dt == F64:
        return np.ascontiguousarray(x, dtype=np.float64)
    if dt == TF32:
        x = np.ascontiguousarray(x)
        if x.dtype != np.float32:
            raise TypeError("tf32 oracle inputs are float32 values")
        return x
    if dt == FP8:
        x = np.ascontiguousarray(x)
        if x.dtype != np.uint8:
            raise TypeError("fp8 oracle inputs are uint8 E4M3 codes")
        return x
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("16-bit oracle inputs are uint16 bit patterns")
    return x


def encode_f16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    _load().oracle_encode_f16_array(_ptr(x), _ptr(y), x.size)
    return y


def encode_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    _load().oracle_encode_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def decode_f16(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, np.float32)
    _load().oracle_decode_f16_array(_ptr(h), _ptr(y), h.size)
    return y


def decode_bf16(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, np.float32)
    _load().oracle_decode_bf16_array(_ptr(h), _ptr(y), h.size)
    return y


def encode_fp8(x):
    """float32 -> fp8 E4M3 codes (nearest-even; NaN beyond 464 in magnitude)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint8)
    _load().oracle_encode_fp8_array(_ptr(x), _ptr(y), x.size)
    return y


def decode_fp8(c):
    c = np.ascontiguousarray(c, dtype=np.uint8)
    y = np.empty(c.shape, np.float32)
    _load().oracle_decode_fp8_array(_ptr(c), _ptr(y), c.size)
    return y


def round_tf32(x):
    """float32 -> float32 rounded to tf32 (10 fraction bits, nearest-even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.float32)
    _load().oracle_round_tf32_array(_ptr(x), _ptr(y), x.size)
    return y


def decode(dtype, x):
    dt = dtype_code(dtype)
    if dt == F64:
        return np.asarray(x, dtype=np.float64)
    if dt == TF32:
        return np.asarray(x, dtype=np.float32)
    if dt == FP8:
        return decode_fp8(x)
    return decode_f16(x) if dt == F16 else decode_bf16(x)


def encode(dtype, x):
    dt = dtype_code(dtype)
    if dt == F64:
        return np.asarray(x, dtype=np.float64)
    if dt == TF32:
        return np.asarray(x, dtype=np.float32)
    if dt == FP8:
        return encode_fp8(x)
    return encode_f16(x) if dt == F16 else encode_bf16(x)


def gemm_acc(dtype, X, B):
    """One stage before rounding: sum_k X[m,k]*B[k,n], k ascending from +0,
    float32 for 16-bit inputs (returned as float32), float64 with fma for fp64,
    float32 over operands rounded to tf32 for tf32."""
    dt = dtype_code(dtype)
    X = _as_input(dt, X)
    B = _as_input(dt, B)
    M, K = X.shape
    K2, N = B.shape
    assert K == K2
    out = np.empty((M, N), np.float64 if dt == F64 else np.float32)     # tf32 sums in float32 too
    rc = _load().oracle_gemm_acc(dt, M, K, N, _ptr(X), _ptr(B), _ptr(out))
    if rc:
        raise ValueError(f"oracle_gemm_acc failed ({rc})")
    return out


def cascade(dtype, A, Bs, rows=None, nthreads=None):
    """D = rnd(...rnd(rnd(A.B0).B1)...) for every batch.

    A: [batch, M, K] (or [M, K]); Bs: list of [batch, d_s, d_{s+1}] (or 2-D).
    16-bit inputs/outputs are uint16 encodings, fp64 is float64.
    rows: optional flat row ids (b*M + m); then the result is [len(rows), N_last]
    in that order, else [batch, M, N_last] (or [M, N_last] for 2-D A).
    dtype may also be a list of len(Bs) + 1 16-bit types, one per stage: A and
    B_s in types[s], the result of GEMM s rounded into types[s + 1], D in the last.
    """
    if isinstance(dtype, (list, tuple)):
        types = [dtype_code(t) for t in dtype]
        if (len(types) != len(Bs) + 1 or any(t in (F64, TF32) for t in types)
                or FP8 in (types[0], types[-1])):
            raise ValueError("one 16-bit type per GEMM (fp8 after the first) and a 16-bit one for D")
        if len(set(types)) == 1:
            return cascade(types[0], A, Bs, rows, nthreads)
    else:
        types = None
    dt = dtype_code(dtype) if types is None else types[0]
    A = _as_input(dt, A)
    squeeze = A.ndim == 2
    if squeeze:
        A = A[None]
        Bs = [b[None] for b in Bs]
    Bs = [_as_input(dt if types is None else types[s], b) for s, b in enumerate(Bs)]
    batch, M, K = A.shape
    dims = [K] + [b.shape[2] for b in Bs]
    for s, b in enumerate(Bs):
        assert b.shape == (batch, dims[s], dims[s + 1]), (b.shape, dims)
    dims_a = np.array(dims, np.int64)
    bptrs = (ctypes.c_void_p * len(Bs))(*[b.ctypes.data for b in Bs])
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.size
    else:
        nrows = batch * M
    out = np.empty((nrows, dims[-1]), {F64: np.float64, TF32: np.float32}.get(dt, np.uint16))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    if types is None:
        rc = _load().oracle_cascade(dt, len(Bs), _ptr(dims_a), batch, M, _ptr(A), bptrs,
                                    _ptr(rows) if rows is not None else None, nrows, _ptr(out),
                                    int(nthreads))
    else:
        ta = np.array(types, np.int32)
        rc = _load().oracle_cascade_typed(_ptr(ta), len(Bs), _ptr(dims_a), batch, M, _ptr(A), bptrs,
                                          _ptr(rows) if rows is not None else None, nrows, _ptr(out),
                                          int(nthreads))
    if rc:
        raise ValueError(f"oracle_cascade failed ({rc})")
    if rows is not None:
        return out
    out = out.reshape(batch, M, dims[-1])
    return out[0] if squeeze else out
