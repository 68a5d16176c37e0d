"""CPU oracle for FP8 quantization and scaled GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding in ``fp8_scaled_matmul_amd``) never imports, links or calls
it, and it never imports the product path.

The arithmetic lives in ``fp8_oracle.c`` (plain C, gcc, no fast-math, no FMA
contraction); this module only builds it and marshals numpy arrays.  Every
definition it follows is cited in ``fp8_oracle.h``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
BF16, FP32 = 0, 1
TENSOR, ROW_1x128, BLOCK_128x128 = 0, 1, 2
FROM_AMAX, GIVEN = 0, 1

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Counters(ctypes.Structure):
    _fields_ = [("saturated", ctypes.c_uint64), ("underflow", ctypes.c_uint64),
                ("nan", ctypes.c_uint64), ("nonfinite_out", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        i64, f32, f64, vp, i32 = (ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                                  ctypes.c_void_p, ctypes.c_int)
        L.orc_decode.restype = f64
        L.orc_decode.argtypes = [i32, ctypes.c_uint8]
        L.orc_fmax.restype = f64
        L.orc_fmax.argtypes = [i32]
        L.orc_encode.restype = ctypes.c_uint8
        L.orc_encode.argtypes = [i32, f32, i32, ctypes.POINTER(i32)]
        L.orc_cast_one.restype = ctypes.c_uint8
        L.orc_cast_one.argtypes = [i32, f32, f32, ctypes.POINTER(Counters)]
        L.orc_scale_from_amax.restype = f32
        L.orc_scale_from_amax.argtypes = [i32, f32]
        L.orc_scale_count.restype = i64
        L.orc_scale_count.argtypes = [i32, i64, i64]
        L.orc_amax.restype = None
        L.orc_amax.argtypes = [vp, i32, i64, i64, i64, i32, vp]
        L.orc_quantize.restype = i32
        L.orc_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, i32, vp,
                                   vp, i64, vp, i64, ctypes.POINTER(Counters)]
        L.orc_gemm.restype = i32
        L.orc_gemm.argtypes = [vp, i32, i64, vp, i32, vp, i32, i64, vp, i32,
                               i64, i64, i64, vp, i64]
        L.orc_gemm_points.restype = i32
        L.orc_gemm_points.argtypes = [vp, i32, i64, vp, i32, vp, i32, i64, vp, i32,
                                      i64, i64, i64, vp, vp, i64, vp]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne.argtypes = [f64]
        L.orc_count_nonfinite_bf16.restype = ctypes.c_uint64
        L.orc_count_nonfinite_bf16.argtypes = [vp, i64]
        L.orc_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return FP32
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32")


def num_threads() -> int:
    return lib().orc_num_threads()


def fmax(fmt: int) -> float:
    return lib().orc_fmax(fmt)


def decode(fmt: int, codes) -> np.ndarray:
    """Real value of each FP8 code (float64)."""
    L = lib()
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([L.orc_decode(fmt, c) for c in range(256)], dtype=np.float64)
    return table[codes]


def encode(fmt: int, v: float, src_nonzero: bool = True) -> tuple[int, int]:
    """(code, event) for one fp32 value already divided by its scale."""
    ev = ctypes.c_int(0)
    code = lib().orc_encode(fmt, float(np.float32(v)), int(src_nonzero), ctypes.byref(ev))
    return int(code), int(ev.value)


def cast_one(fmt: int, x: float, s: float) -> tuple[int, dict]:
    c = Counters()
    code = lib().orc_cast_one(fmt, float(np.float32(x)), float(np.float32(s)), ctypes.byref(c))
    return int(code), c.as_dict()


def scale_from_amax(fmt: int, amax: float) -> np.float32:
    return np.float32(lib().orc_scale_from_amax(fmt, float(np.float32(amax))))


def scale_count(gran: int, rows: int, cols: int) -> int:
    return int(lib().orc_scale_count(gran, rows, cols))


def scale_shape(gran: int, rows: int, cols: int) -> tuple[int, ...]:
    nt = -(-cols // 128)
    if gran == TENSOR:
        return (1,)
    if gran == ROW_1x128:
        return (rows, nt)
    return (-(-rows // 128), nt)


def amax(x: np.ndarray, gran: int = TENSOR) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    out = np.zeros(scale_shape(gran, rows, cols), dtype=np.float32)
    lib().orc_amax(_ptr(x), _dtype_code(x), rows, cols, cols, gran, _ptr(out))
    return out


def quantize(x: np.ndarray, fmt: int, gran: int = TENSOR, mode: int = FROM_AMAX,
             scale: np.ndarray | None = None, want_t: bool = False):
    """Returns (q [rows,cols] uint8, q_t [cols,rows] uint8 or None,
    scale float32 array, counters dict)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if mode == GIVEN:
        s = np.ascontiguousarray(np.asarray(scale, dtype=np.float32).reshape(scale_shape(gran, rows, cols)))
    else:
        s = np.zeros(scale_shape(gran, rows, cols), dtype=np.float32)
    q = np.empty((rows, cols), dtype=np.uint8)
    qt = np.empty((cols, rows), dtype=np.uint8) if want_t else None
    c = Counters()
    rc = lib().orc_quantize(_ptr(x), _dtype_code(x), rows, cols, cols, fmt, gran, mode,
                            _ptr(s), _ptr(q), cols, _ptr(qt), rows, ctypes.byref(c))
    if rc != 0:
        raise ValueError("oracle quantize rejected its arguments")
    return q, qt, s, c.as_dict()


def _scale_arr(s, gran, rows, k):
    if gran == TENSOR:
        return np.ascontiguousarray(np.asarray(s, dtype=np.float32).reshape(1))
    return np.ascontiguousarray(np.asarray(s, dtype=np.float32))


def gemm(a: np.ndarray, fa: int, sa, ga: int, b: np.ndarray, fb: int, sb, gb: int) -> np.ndarray:
    """y = (s_a A)(s_b B)^T in fp64, TN layout: a [m,k], b [n,k]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    sa_ = _scale_arr(sa, ga, m, k)
    sb_ = _scale_arr(sb, gb, n, k)
    y = np.empty((m, n), dtype=np.float64)
    rc = lib().orc_gemm(_ptr(a), fa, k, _ptr(sa_), ga, _ptr(b), fb, k, _ptr(sb_), gb,
                        m, n, k, _ptr(y), n)
    if rc != 0:
        raise ValueError("oracle gemm rejected its arguments")
    return y


def gemm_points(a: np.ndarray, fa: int, sa, ga: int, b: np.ndarray, fb: int, sb, gb: int,
                pm: np.ndarray, pn: np.ndarray) -> np.ndarray:
    """The same definition at selected output positions only."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    m, k = a.shape
    n, _ = b.shape
    sa_ = _scale_arr(sa, ga, m, k)
    sb_ = _scale_arr(sb, gb, n, k)
    pm = np.ascontiguousarray(pm, dtype=np.int64)
    pn = np.ascontiguousarray(pn, dtype=np.int64)
    out = np.empty(pm.shape[0], dtype=np.float64)
    rc = lib().orc_gemm_points(_ptr(a), fa, k, _ptr(sa_), ga, _ptr(b), fb, k, _ptr(sb_), gb,
                               m, n, k, _ptr(pm), _ptr(pn), pm.shape[0], _ptr(out))
    if rc != 0:
        raise ValueError("oracle gemm_points rejected its arguments")
    return out


def bf16_rne(y) -> np.ndarray:
    """bf16 bit patterns of real values, RNE."""
    L = lib()
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    out = np.fromiter((L.orc_bf16_rne(float(v)) for v in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(y.shape)


def count_nonfinite_bf16(y: np.ndarray) -> int:
    y = np.ascontiguousarray(y, dtype=np.float64)
    return int(lib().orc_count_nonfinite_bf16(_ptr(y), y.size))


def requant(master: np.ndarray, fmt: int, gran: int = TENSOR, want_t: bool = True):
    """The weight-copy cache refresh after an optimizer step ("#84 FP8
    Precision", section "Hardware precision": the FP8 copy is rebuilt from the
    bf16 master after every step and kept for the next forward pass).  By
    definition it is a fresh quantize of the current master with a current
    amax scale."""
    return quantize(master, fmt, gran, FROM_AMAX, None, want_t)


def quantize_delayed(x: np.ndarray, fmt: int, history, pos: int, want_t: bool = False):
    """Per-tensor quantize with delayed scaling and an amax history ("FP8
    stability guardrails", section "Real products": delayed scaling with
    amax history tracking, the standard FP8 workflow of Transformer Engine).

    Reading taken (the pages name the method only): the history holds the
    amax values of the last len(history) steps.  The tensor is cast with
    the scale the current-scaling rule gives for the LARGEST recorded amax
    (so the tensor's own amax does not enter its own cast), then its amax
    replaces the entry at `pos`, the oldest one, and `pos` advances
    cyclically.  Entries are finite and >= 0; an all-zero history gives
    s = 1, as amax == 0 does.

    Returns (q, q_t or None, scale float32 [1], counters dict,
    new history float32 array, new pos)."""
    h = np.asarray(history, dtype=np.float32).reshape(-1)
    if h.size < 1 or not (0 <= pos < h.size):
        raise ValueError("history needs >= 1 entry and 0 <= pos < len(history)")
    s = scale_from_amax(fmt, float(h.max()))
    q, qt, s_arr, ctr = quantize(x, fmt, TENSOR, GIVEN, np.array([s], dtype=np.float32), want_t)
    new = h.copy()
    new[pos] = amax(x, TENSOR)[0]
    return q, qt, s_arr, ctr, new, (pos + 1) % h.size


def scale_pow2(fmt: int, amax: float) -> np.float32:
    """Power-of-two scale of a group: the smallest s = 2^e (e an integer)
    with amax / s <= fmax, taken on the real quotient; amax == 0 gives 1 and
    e is raised to -126 (s stays a normal fp32 number, and its exponent field
    is the E8M0 code the gfx950 scaled MFMA takes).  Not on the pages: the
    MI355X-native form of their fine-grained tile and block scaling ("FP8
    stability guardrails", section "Real products"), with the scale
    restricted to powers of two so that the matrix core can apply it."""
    a = float(np.float32(amax))
    if not a > 0.0:
        return np.float32(1.0)
    f = fmax(fmt)
    e = math.frexp(a)[1] - math.frexp(f)[1]
    while math.ldexp(f, e) < a:          # exact products of a power of two
        e += 1
    while math.ldexp(f, e - 1) >= a:
        e -= 1
    return np.float32(math.ldexp(1.0, max(e, -126)))


def quantize_pow2(x: np.ndarray, fmt: int, gran: int = TENSOR, want_t: bool = False):
    """Quantize with power-of-two scales: per group, amax (as for FROM_AMAX),
    s = scale_pow2(amax), then the cast of the GIVEN mode with those scales.
    Returns (q, q_t or None, scale float32 array, counters dict)."""
    a = amax(x, gran)
    s = np.array([scale_pow2(fmt, v) for v in a.reshape(-1)], dtype=np.float32).reshape(a.shape)
    return quantize(x, fmt, gran, GIVEN, s, want_t)

