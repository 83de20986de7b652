"""Python binding of libb2b.so, the fused cascaded-GEMM library for MI355X.

Argument marshalling only: every step of the cascade runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  torch is
imported before the library is loaded so that both share one HIP runtime.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libb2b.so")

F16, BF16, F64, TF32, FP8 = 0, 1, 2, 3, 4
DTYPES = {"f16": F16, "bf16": BF16, "f64": F64, "tf32": TF32, "fp8": FP8}
# tf32 cascades take and return float32 tensors (the GEMMs round their operands to tf32)
TORCH_DTYPES = {F16: torch.float16, BF16: torch.bfloat16, F64: torch.float64, TF32: torch.float32}
REMAP = {"auto": 0, "bpermute": 1, "permlane": 2, "lds": 3, "relabel": 4}
FLAG_UNFUSED, FLAG_ORIENT_N, FLAG_MFMA_32X32, FLAG_TF32_EXACT = 1, 2, 4, 8
SHAPES = {"f16_16x16x32": 0, "bf16_16x16x32": 1, "f16_32x32x16": 2, "bf16_32x32x16": 3,
          "f16_16x16x16": 4, "f64_16x16x4": 5, "fp8_32x32x64": 6}
STATUS = {0: "success", 1: "invalid value", 2: "not supported", 3: "HIP runtime error",
          4: "out of memory", 5: "intermediates exceed the static workspace"}
STATIC_WORKSPACE_BYTES = 32 << 20
EXPORTS = ("b2b_gemm_create", "b2b_gemm_run", "b2b_chain_create", "b2b_chain_create_typed", "b2b_chain_run", "b2b_chain_run_static", "b2b_gemm_tune",
           "b2b_gemm_destroy", "b2b_status_string",
           "b2b_gemm_get_info", "b2b_remap_relation", "b2b_remap_schedule", "b2b_remap_compile",
           "b2b_remap_execute", "b2b_remap_probe",
           "b2b_mfma_probe", "b2b_fp8_convert_probe")
# measurement instruments (b2b_bench.h)
BENCH_EXPORTS = ("b2b_bench_mfma", "b2b_bench_copy", "b2b_bench_stream")


class B2BError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m chip_fusion_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, u32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
        L.b2b_gemm_create.argtypes = [ctypes.POINTER(vp), i32, i64, i64, i64, i64, i64, i64,
                                      ctypes.POINTER(i64), ctypes.POINTER(i64), u32]
        L.b2b_gemm_run.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.b2b_chain_create.argtypes = [ctypes.POINTER(vp), i32, i64, i64, ctypes.c_int32, ctypes.POINTER(i64),
                                       ctypes.POINTER(i64), ctypes.POINTER(i64), u32]
        L.b2b_chain_run.argtypes = [vp, vp, ctypes.POINTER(vp), vp, vp]
        L.b2b_chain_run_static.argtypes = [i32, i64, i64, ctypes.c_int32, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                           ctypes.POINTER(i64), vp, ctypes.POINTER(vp), vp, vp]
        L.b2b_chain_create_typed.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i32), i64, i64, ctypes.c_int32,
                                             ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64), u32]
        L.b2b_chain_create_typed.restype = i32
        L.b2b_gemm_tune.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    ctypes.POINTER(vp), vp, ctypes.c_int32]
        L.b2b_gemm_destroy.argtypes = [vp]
        L.b2b_status_string.argtypes = [i32]
        L.b2b_status_string.restype = ctypes.c_char_p
        L.b2b_gemm_get_info.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
        L.b2b_remap_relation.argtypes = [i32, i32, vp, i64, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_int32)]
        L.b2b_remap_schedule.argtypes = [i32, i32, i32, vp, vp, vp, i64, ctypes.POINTER(ctypes.c_int32)]
        L.b2b_remap_probe.argtypes = [i32, i32, u32, vp, vp, vp]
        L.b2b_remap_compile.argtypes = [i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_int32)]
        L.b2b_remap_execute.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp]
        L.b2b_mfma_probe.argtypes = [i32, vp, vp, vp, vp]
        L.b2b_fp8_convert_probe.argtypes = [vp, vp, vp]
        L.b2b_bench_mfma.argtypes = [i32, i32, i64, vp, ctypes.POINTER(ctypes.c_double), vp]
        L.b2b_bench_copy.argtypes = [vp, vp, i64, i32, vp]
        L.b2b_bench_stream.argtypes = [vp, i64, vp, i64, i32, vp]
        for n in EXPORTS + BENCH_EXPORTS:
            if n not in ("b2b_status_string",):
                getattr(L, n).restype = i32
        _lib = L
    return _lib


def _check(st, what):
    if st != 0:
        raise B2BError(st, what)


def _stream_ptr(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _torch_dtype(code):
    return torch.uint8 if code == FP8 else TORCH_DTYPES[code]


def _dense(widths, batch, M, ld, batch_stride):
    """Leading dimensions and batch strides of every operand (A, B_0..B_{n-1},
    D), as the library takes them: the given ones, or the dense defaults."""
    rows = [M] + list(widths[:-1]) + [M]
    width = [widths[0]] + list(widths[1:]) + [widths[-1]]
    L = list(ld) if ld is not None else width
    S = list(batch_stride) if batch_stride is not None else [r * l for r, l in zip(rows, L)]
    return rows, width, L, S


def _check_operand(t, name, dtype, batch, rows, width, ld, bs):
    """Raises ValueError unless tensor t can hold operand `name` as the plan
    addresses it: a device tensor of the plan's type whose memory from its
    first element covers (batch - 1) * bs + (rows - 1) * ld + width elements.
    The kernels address by the plan's sizes, not by the tensor's shape, so a
    smaller tensor would be read or written past its end."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: a torch tensor is expected, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {dtype} expected, got {t.dtype}")
    need = (batch - 1) * bs + (rows - 1) * ld + width
    have = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if have < need:
        raise ValueError(f"{name}: the plan addresses {need} elements from its first one, "
                         f"the tensor's memory holds {have}")


class Plan:
    """A planned cascade D = rnd(rnd(A.B0).B1)[.B2] (b2b_gemm_create)."""

    def __init__(self, dtype, batch, M, K, N1, N2, N3=0, ld=None, batch_stride=None,
                 remap="auto", orient_n=False, unfused=False, mfma32=False, tf32_exact=False):
        self.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
        self.batch, self.M, self.dims = batch, M, [K, N1, N2] + ([N3] if N3 else [])
        flags = ((REMAP[remap] << 4) | (FLAG_ORIENT_N if orient_n else 0) | (FLAG_UNFUSED if unfused else 0)
                 | (FLAG_MFMA_32X32 if mfma32 else 0) | (FLAG_TF32_EXACT if tf32_exact else 0))
        arr = ctypes.c_int64 * 5
        h = ctypes.c_void_p()
        st = lib().b2b_gemm_create(ctypes.byref(h), self.dtype, batch, M, K, N1, N2, N3,
                                   arr(*ld) if ld is not None else None,
                                   arr(*batch_stride) if batch_stride is not None else None, flags)
        _check(st, "b2b_gemm_create")
        self._h = h
        nst = len(self.dims) - 1
        if ld is not None or batch_stride is not None:
            pick = lambda v: None if v is None else [v[i] for i in range(5) if not (i == 3 and nst == 2)]
            ld, batch_stride = pick(ld), pick(batch_stride)
        self._layout = _dense(self.dims, batch, M, ld, batch_stride)
        self._types = [self.dtype] * (nst + 1)

    def _check_tensors(self, A, Bs, D):
        """ValueError before any launch if a tensor does not fit the plan."""
        rows, width, L, S = self._layout
        nst = len(self.dims) - 1
        if len(Bs) != nst:
            raise ValueError(f"{nst} weight matrices expected, got {len(Bs)}")
        ts = self._types
        ops = [("A", A, ts[0])] + [(f"B{i}", b, ts[i]) for i, b in enumerate(Bs)] + [("D", D, ts[-1])]
        for i, (name, t, code) in enumerate(ops):
            _check_operand(t, name, _torch_dtype(code), self.batch, rows[i], width[i], L[i], S[i])
        for name, t, _ in ops:
            if t.device.type != "cuda":
                raise ValueError(f"{name}: a device (cuda) tensor is expected, got one on {t.device}")

    def run(self, A, B0, B1, B2=None, D=None, stream=None):
        if D is None:
            D = torch.empty((self.batch, self.M, self.dims[-1]), dtype=A.dtype, device=A.device)
        self._check_tensors(A, [B0, B1] + ([B2] if B2 is not None else []), D)
        st = lib().b2b_gemm_run(self._h, _ptr(A), _ptr(B0), _ptr(B1), _ptr(B2), _ptr(D),
                                _stream_ptr(stream))
        _check(st, "b2b_gemm_run")
        return D

    def tune(self, sets, reps=10, stream=None):
        """Keeps the fastest compiled kernel for this cascade (b2b_gemm_tune),
        timed over `sets`, a list of (A, [B_0, ..], D) representative of the
        use; every D holds the kept kernel's result afterwards."""
        nst = len(self.dims) - 1
        for a, Bs, d in sets:
            self._check_tensors(a, list(Bs), d)
        n = len(sets)
        As = (ctypes.c_void_p * n)(*[a.data_ptr() for a, _, _ in sets])
        Bp = (ctypes.c_void_p * (n * nst))(*[b.data_ptr() for _, Bs, _ in sets for b in Bs])
        Ds = (ctypes.c_void_p * n)(*[d.data_ptr() for _, _, d in sets])
        _check(lib().b2b_gemm_tune(self._h, n, As, Bp, Ds, _stream_ptr(stream), reps), "b2b_gemm_tune")

    def info(self):
        buf = ctypes.create_string_buffer(512)
        _check(lib().b2b_gemm_get_info(self._h, buf, 512), "b2b_gemm_get_info")
        return buf.value.decode()

    def close(self):
        if getattr(self, "_h", None):
            lib().b2b_gemm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Chain(Plan):
    """A planned cascade of any number of GEMMs (b2b_chain_create):
    D = rnd(...rnd(A.B_0)...B_{n-1}) with widths [K, N_1, ..., N_n].
    dtype may be a list of len(widths) types, one per GEMM and the last for D
    (b2b_chain_create_typed)."""

    def __init__(self, dtype, batch, M, widths, ld=None, batch_stride=None, remap="auto",
                 unfused=False, mfma32=False, tf32_exact=False):
        code = lambda t: DTYPES[t] if isinstance(t, str) else int(t)
        typed = isinstance(dtype, (list, tuple))
        self.dtypes = [code(t) for t in dtype] if typed else None
        self.dtype = self.dtypes[0] if typed else code(dtype)
        self.batch, self.M, self.dims = batch, M, list(widths)
        nst = len(self.dims) - 1
        flags = ((REMAP[remap] << 4) | (FLAG_UNFUSED if unfused else 0) | (FLAG_MFMA_32X32 if mfma32 else 0)
                 | (FLAG_TF32_EXACT if tf32_exact else 0))
        w = (ctypes.c_int64 * (nst + 1))(*self.dims)
        arr = ctypes.c_int64 * (nst + 2)
        h = ctypes.c_void_p()
        lds = arr(*ld) if ld is not None else None
        bss = arr(*batch_stride) if batch_stride is not None else None
        if typed:
            if len(self.dtypes) != nst + 1:
                raise ValueError(f"{nst + 1} types expected (one per GEMM and D), got {len(self.dtypes)}")
            ts = (ctypes.c_int32 * (nst + 1))(*self.dtypes)
            st = lib().b2b_chain_create_typed(ctypes.byref(h), ts, batch, M, nst, w, lds, bss, flags)
            _check(st, "b2b_chain_create_typed")
        else:
            st = lib().b2b_chain_create(ctypes.byref(h), self.dtype, batch, M, nst, w, lds, bss, flags)
            _check(st, "b2b_chain_create")
        self._h = h
        self._layout = _dense(self.dims, batch, M, ld, batch_stride)
        self._types = list(self.dtypes) if typed else [self.dtype] * (nst + 1)

    def run(self, A, *Bs, D=None, stream=None):
        if len(Bs) != len(self.dims) - 1:
            raise ValueError(f"{len(self.dims) - 1} weight matrices expected, got {len(Bs)}")
        if D is None:
            dt = TORCH_DTYPES[self.dtypes[-1]] if self.dtypes else A.dtype
            D = torch.empty((self.batch, self.M, self.dims[-1]), dtype=dt, device=A.device)
        self._check_tensors(A, list(Bs), D)
        ptrs = (ctypes.c_void_p * len(Bs))(*[b.data_ptr() for b in Bs])
        st = lib().b2b_chain_run(self._h, _ptr(A), ptrs, _ptr(D), _stream_ptr(stream))
        _check(st, "b2b_chain_run")
        return D


def chain_run_static(dtype, batch, M, widths, A, Bs, D, ld=None, batch_stride=None, stream=None):
    """The unfused cascade with the library's static workspace
    (b2b_chain_run_static): nothing is allocated by the call."""
    code = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    widths = list(widths)
    nst = len(widths) - 1
    if len(Bs) != nst:
        raise ValueError(f"{nst} weight matrices expected, got {len(Bs)}")
    rows, width, L, S = _dense(widths, batch, M, ld, batch_stride)
    ops = [("A", A)] + [(f"B{i}", b) for i, b in enumerate(Bs)] + [("D", D)]
    for i, (name, t) in enumerate(ops):
        _check_operand(t, name, _torch_dtype(code), batch, rows[i], width[i], L[i], S[i])
    for name, t in ops:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: a device (cuda) tensor is expected, got one on {t.device}")
    arr = ctypes.c_int64 * (nst + 2)
    w = (ctypes.c_int64 * (nst + 1))(*widths)
    ptrs = (ctypes.c_void_p * nst)(*[b.data_ptr() for b in Bs])
    st = lib().b2b_chain_run_static(code, batch, M, nst, w, arr(*ld) if ld is not None else None,
                                    arr(*batch_stride) if batch_stride is not None else None, _ptr(A), ptrs,
                                    _ptr(D), _stream_ptr(stream))
    _check(st, "b2b_chain_run_static")
    return D


def _need(t, nbytes, name):
    """ValueError unless t is a contiguous device tensor of at least nbytes:
    the probe kernels read and write fixed sizes, whatever the tensor holds."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{name}: a contiguous device tensor is expected")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {nbytes} bytes expected, the tensor holds {t.numel() * t.element_size()}")


def remap_relation(shape, orient_n=False):
    """Relation table of one remap unit and elements per lane (b2b_remap_relation)."""
    sh = SHAPES[shape] if isinstance(shape, str) else shape
    n = ctypes.c_int64()
    e = ctypes.c_int32()
    _check(lib().b2b_remap_relation(sh, int(orient_n), None, 0, ctypes.byref(n), ctypes.byref(e)),
           "b2b_remap_relation")
    out = np.empty(n.value, np.int32)
    _check(lib().b2b_remap_relation(sh, int(orient_n), out.ctypes.data, n.value, ctypes.byref(n),
                                    ctypes.byref(e)), "b2b_remap_relation")
    return out, e.value


def remap_schedule(shape, orient_n=False, packed=False):
    """Coordination rounds (p, q, r), each [rounds, 64] (b2b_remap_schedule)."""
    sh = SHAPES[shape] if isinstance(shape, str) else shape
    rounds = ctypes.c_int32()
    _check(lib().b2b_remap_schedule(sh, int(orient_n), int(packed), None, None, None, 0,
                                    ctypes.byref(rounds)), "b2b_remap_schedule")
    n = rounds.value * 64
    p, q, r = (np.empty(n, np.int32) for _ in range(3))
    _check(lib().b2b_remap_schedule(sh, int(orient_n), int(packed), p.ctypes.data, q.ctypes.data,
                                    r.ctypes.data, n, ctypes.byref(rounds)), "b2b_remap_schedule")
    return p.reshape(-1, 64), q.reshape(-1, 64), r.reshape(-1, 64)


def remap_compile(src, dst):
    """Relation and coordination rounds between two layouts given as labels
    [64 * E] (b2b_remap_compile); returns rel, p, q, r ([E, 64] each for p, q, r)."""
    src = np.ascontiguousarray(src, np.int32)
    dst = np.ascontiguousarray(dst, np.int32)
    if src.size != dst.size or src.size % 64:
        raise ValueError("layouts must hold 64 * E labels each")
    E = src.size // 64
    rel = np.empty(src.size, np.int32)
    p, q, r = (np.empty(src.size, np.int32) for _ in range(3))
    rounds = ctypes.c_int32()
    _check(lib().b2b_remap_compile(E, src.ctypes.data, dst.ctypes.data, rel.ctypes.data, p.ctypes.data,
                                   q.ctypes.data, r.ctypes.data, ctypes.byref(rounds)), "b2b_remap_compile")
    return rel, p.reshape(E, 64), q.reshape(E, 64), r.reshape(E, 64)


def remap_execute(p, q, r, payload, stream=None):
    """Runs compiled rounds on a device int32/uint32 tensor [64 * E] (b2b_remap_execute)."""
    p, q, r = (np.ascontiguousarray(x, np.int32).reshape(-1) for x in (p, q, r))
    E = p.size // 64
    if p.size % 64 or q.size != p.size or r.size != p.size:
        raise ValueError("p, q, r: [E, 64] each")
    if payload.dtype not in (torch.int32, torch.uint32) or payload.numel() != 64 * E:
        raise ValueError(f"payload: 64 * E = {64 * E} 32-bit values expected")
    _need(payload, 256 * E, "payload")
    out = torch.empty_like(payload)
    _check(lib().b2b_remap_execute(E, E, p.ctypes.data, q.ctypes.data, r.ctypes.data, _ptr(payload), _ptr(out),
                                   _stream_ptr(stream)), "b2b_remap_execute")
    return out


def remap_probe(shape, mode, inp, orient_n=False, stream=None):
    """Runs the device rearrangement executor `mode` on payload tensor `inp`."""
    sh = SHAPES[shape] if isinstance(shape, str) else shape
    _need(inp, 2048 if sh == SHAPES["f64_16x16x4"] else 1024, "inp")   # 4 doubles or 8 16-bit values a lane
    out = torch.empty_like(inp)
    st = lib().b2b_remap_probe(sh, int(orient_n), REMAP[mode] << 4, _ptr(inp), _ptr(out),
                               _stream_ptr(stream))
    _check(st, "b2b_remap_probe")
    return out


def mfma_probe(shape, a, b, stream=None):
    """One matrix instruction on raw operands a, b ([64, elems] device tensors);
    returns the accumulator registers, [64, 4] ([64, 16] for 32x32x16) (b2b_mfma_probe)."""
    sh = SHAPES[shape] if isinstance(shape, str) else shape
    acc_dtype = torch.float64 if a.dtype == torch.float64 else torch.float32
    nacc = 16 if sh in (SHAPES["f16_32x32x16"], SHAPES["bf16_32x32x16"], SHAPES["fp8_32x32x64"]) else 4
    per_lane = 8 if sh == SHAPES["f64_16x16x4"] else (32 if sh == SHAPES["fp8_32x32x64"] else 16)
    _need(a, 64 * per_lane, "a")
    _need(b, 64 * per_lane, "b")
    c = torch.empty((64, nacc), dtype=acc_dtype, device=a.device)
    _check(lib().b2b_mfma_probe(sh, _ptr(a), _ptr(b), _ptr(c), _stream_ptr(stream)), "b2b_mfma_probe")
    return c


def fp8_convert_probe(x, stream=None):
    """The kernels' fp32 -> fp8 E4M3 conversion of 256 values (a float32
    device tensor); returns the 256 codes as a uint8 device tensor."""
    if x.numel() != 256 or x.dtype != torch.float32:
        raise ValueError("256 float32 values expected")
    y = torch.empty(256, dtype=torch.uint8, device=x.device)
    _check(lib().b2b_fp8_convert_probe(_ptr(x), _ptr(y), _stream_ptr(stream)), "b2b_fp8_convert_probe")
    return y


def bench_mfma(dtype, workgroups, iters, sink, stream=None):
    """Enqueues the matrix-core-only loop (b2b_bench_mfma) on a float64
    device tensor `sink` of workgroups * 256 values; returns its FLOP."""
    if sink.dtype != torch.float64 or sink.numel() < workgroups * 256 or sink.device.type != "cuda":
        raise ValueError("sink: a float64 device tensor of workgroups * 256 values is expected")
    flop = ctypes.c_double()
    _check(lib().b2b_bench_mfma(DTYPES[dtype], workgroups, iters, _ptr(sink), ctypes.byref(flop),
                                _stream_ptr(stream)), "b2b_bench_mfma")
    return flop.value


def _stream_operands(src, dst):
    for name, x in (("src", src), ("dst", dst)):
        if x.device.type != "cuda" or not x.is_contiguous():
            raise ValueError(f"{name}: a contiguous device tensor is expected")
    return src.numel() * src.element_size(), dst.numel() * dst.element_size()


def bench_copy(src, dst, workgroups, stream=None):
    """Enqueues the HBM stream dst = src over all of src's bytes (b2b_bench_copy)."""
    n, m = _stream_operands(src, dst)
    if m < n:
        raise ValueError("dst must be at least as large as src")
    _check(lib().b2b_bench_copy(_ptr(src), _ptr(dst), n, workgroups, _stream_ptr(stream)), "b2b_bench_copy")


def bench_stream(src, dst, workgroups, stream=None):
    """Enqueues the mixed stream (b2b_bench_stream): all of src's bytes read as
    R back-to-back streams, XOR-folded into all of dst's bytes, R = src bytes /
    dst bytes (an integer, 1 to 4)."""
    n, m = _stream_operands(src, dst)
    if m < 64 or n % m or not 1 <= n // m <= 4:
        raise ValueError("src must hold 1 to 4 times dst's bytes, dst at least 64 bytes")
    _check(lib().b2b_bench_stream(_ptr(src), n, _ptr(dst), m, workgroups, _stream_ptr(stream)),
           "b2b_bench_stream")


def to_device(x, dtype, device="cuda"):
    """numpy input (uint16 encodings, float64, float32 for tf32, uint8 codes
    for fp8) -> torch tensor of the dtype (fp8: uint8)."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    if dt == F64:
        return torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(device)
    if dt == TF32:
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
    if dt == FP8:
        return torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(TORCH_DTYPES[dt])
    return t.to(device)


def to_host(t):
    """torch tensor -> numpy (uint16 encodings for 16-bit types, float64, float32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float64, torch.float32):
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)
