"""Python binding of the MI355X FP8 scaled-matmul library (libfp8mi.so).

Argument marshalling only: every step of quantization, GEMM and cache refresh
runs in the HIP kernels behind the C ABI declared in include/fp8mi.h.  Torch
supplies device memory and the current stream; nothing here computes.

The functions named ``fp8_*`` mirror the C entry points one to one (raw
device pointers as ints).  The tensor-level helpers (``quantize``,
``scaled_mm``, ``WeightCache`` ...) allocate outputs and workspaces with torch
and call those.

If the library has not been built, importing works but every call raises
``RuntimeError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfp8mi.so")

# enums of include/fp8mi.h
FP8_OK, FP8_ERR_INVALID_ARG, FP8_ERR_UNSUPPORTED_SHAPE, FP8_ERR_UNSUPPORTED_DEVICE, FP8_ERR_HIP = range(5)
E4M3, E5M2 = 0, 1
BF16, FP32 = 0, 1
TENSOR, ROW_1x128, BLOCK_128x128 = 0, 1, 2
ROW_1x128_POW2, BLOCK_128x128_POW2 = 3, 4      # GEMM operands with power-of-two scales
FROM_AMAX, GIVEN, FROM_AMAX_POW2 = 0, 1, 2

EXPORTED = [
    "fp8_abi_version", "fp8_status_string", "fp8_last_error",
    "fp8_amax_workspace_size", "fp8_amax",
    "fp8_quantize_workspace_size", "fp8_quantize", "fp8_quantize_noalloc",
    "fp8_quantize_delayed_workspace_size", "fp8_quantize_delayed",
    "fp8_scaled_mm_workspace_size", "fp8_scaled_mm",
    "fp8_quantize_scaled_mm_workspace_size", "fp8_quantize_scaled_mm",
    "fp8_requant_workspace_size", "fp8_requant_weights",
    "fp8_counters_reset", "fp8_debug_set_wait_limit",
]


class Fp8Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status


class WeightCacheDesc(ctypes.Structure):
    """fp8_weight_cache of include/fp8mi.h."""
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("fmt", ctypes.c_int), ("gran", ctypes.c_int),
                ("q", ctypes.c_void_p), ("q_t", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("ctr", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libfp8mi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp8_scaled_matmul_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.fp8_abi_version.restype = ctypes.c_int32
        L.fp8_abi_version.argtypes = []
        L.fp8_status_string.restype = ctypes.c_char_p
        L.fp8_status_string.argtypes = [i32]
        L.fp8_last_error.restype = ctypes.c_char_p
        L.fp8_last_error.argtypes = []
        L.fp8_amax_workspace_size.restype = sz
        L.fp8_amax_workspace_size.argtypes = [i64, i64, i32]
        L.fp8_amax.restype = i32
        L.fp8_amax.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, sz, vp]
        L.fp8_quantize_workspace_size.restype = sz
        L.fp8_quantize_workspace_size.argtypes = [i64, i64, i32, i32]
        L.fp8_quantize.restype = i32
        L.fp8_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, i32, vp,
                                   vp, i64, vp, i64, vp, vp, sz, vp]
        L.fp8_quantize_noalloc.restype = i32
        L.fp8_quantize_noalloc.argtypes = [vp, i32, i64, i64, i64, i32, i32, i32, vp,
                                           vp, i64, vp, i64, vp, vp]
        L.fp8_quantize_delayed_workspace_size.restype = sz
        L.fp8_quantize_delayed_workspace_size.argtypes = [i64, i64]
        L.fp8_quantize_delayed.restype = i32
        L.fp8_quantize_delayed.argtypes = [vp, i32, i64, i64, i64, i32, vp, vp, i32, vp,
                                           vp, i64, vp, i64, vp, vp, sz, vp]
        L.fp8_scaled_mm_workspace_size.restype = sz
        L.fp8_scaled_mm_workspace_size.argtypes = [i64, i64, i64, i32, i32]
        L.fp8_scaled_mm.restype = i32
        L.fp8_scaled_mm.argtypes = [vp, i32, i64, vp, i32, vp, i32, i64, vp, i32,
                                    i64, i64, i64, vp, i64, vp, sz, vp, vp]
        L.fp8_quantize_scaled_mm_workspace_size.restype = sz
        L.fp8_quantize_scaled_mm_workspace_size.argtypes = [i64, i64, i64]
        L.fp8_quantize_scaled_mm.restype = i32
        L.fp8_quantize_scaled_mm.argtypes = [vp, i64, i32, vp, vp, i64, vp, i64, vp, i32, i64, vp,
                                             i64, i64, i64, vp, i64, vp, vp, sz, vp]
        L.fp8_requant_workspace_size.restype = sz
        L.fp8_requant_workspace_size.argtypes = [ctypes.POINTER(WeightCacheDesc), ctypes.c_int32]
        L.fp8_requant_weights.restype = i32
        L.fp8_requant_weights.argtypes = [ctypes.POINTER(WeightCacheDesc), ctypes.POINTER(vp),
                                          ctypes.POINTER(ctypes.c_int), ctypes.c_int32, vp, sz, vp]
        L.fp8_counters_reset.restype = i32
        L.fp8_counters_reset.argtypes = [vp, vp]
        L.fp8_debug_set_wait_limit.restype = ctypes.c_int32
        L.fp8_debug_set_wait_limit.argtypes = [ctypes.c_int32]
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().fp8_status_string(s).decode()
    except Exception:
        return f"status {s}"


def check(status: int) -> None:
    if status != FP8_OK:
        raise Fp8Error(status, lib().fp8_last_error().decode())


# ---------------------------------------------------------------- raw C entry points
def fp8_abi_version() -> int:
    return lib().fp8_abi_version()


def fp8_amax(x, dtype, rows, cols, ld, gran, amax, workspace, workspace_bytes, stream) -> int:
    return lib().fp8_amax(x, dtype, rows, cols, ld, gran, amax, workspace, workspace_bytes, stream)


def fp8_quantize(x, dtype, rows, cols, ld, fmt, gran, mode, scale, q, ldq, q_t, ldq_t, ctr,
                 workspace, workspace_bytes, stream) -> int:
    return lib().fp8_quantize(x, dtype, rows, cols, ld, fmt, gran, mode, scale, q, ldq, q_t, ldq_t, ctr,
                              workspace, workspace_bytes, stream)


def fp8_quantize_noalloc(x, dtype, rows, cols, ld, fmt, gran, mode, scale, q, ldq, q_t, ldq_t, ctr,
                         stream) -> int:
    return lib().fp8_quantize_noalloc(x, dtype, rows, cols, ld, fmt, gran, mode, scale, q, ldq, q_t, ldq_t, ctr,
                                      stream)


def fp8_quantize_delayed(x, dtype, rows, cols, ld, fmt, history, pos, history_len, scale, q, ldq, q_t, ldq_t,
                         ctr, workspace, workspace_bytes, stream) -> int:
    return lib().fp8_quantize_delayed(x, dtype, rows, cols, ld, fmt, history, pos, history_len, scale, q, ldq,
                                      q_t, ldq_t, ctr, workspace, workspace_bytes, stream)


def fp8_scaled_mm(a, fa, lda, scale_a, ga, b, fb, ldb, scale_b, gb, m, n, k, c, ldc,
                  workspace, workspace_bytes, ctr, stream) -> int:
    return lib().fp8_scaled_mm(a, fa, lda, scale_a, ga, b, fb, ldb, scale_b, gb, m, n, k, c, ldc,
                               workspace, workspace_bytes, ctr, stream)


def fp8_quantize_scaled_mm(x, ldx, fa, scale_a, xq, ldxq, xq_t, ldxq_t, b, fb, ldb, scale_b, m, n, k, c, ldc,
                           ctr, workspace, workspace_bytes, stream) -> int:
    return lib().fp8_quantize_scaled_mm(x, ldx, fa, scale_a, xq, ldxq, xq_t, ldxq_t, b, fb, ldb, scale_b, m, n, k,
                                        c, ldc, ctr, workspace, workspace_bytes, stream)


def fp8_requant_weights(descs, masters, dtypes, workspace, workspace_bytes, stream) -> int:
    n = len(descs)
    arr = (WeightCacheDesc * n)(*descs)
    mp = (ctypes.c_void_p * n)(*masters)
    dt = (ctypes.c_int * n)(*dtypes)
    return lib().fp8_requant_weights(arr, mp, dt, n, workspace, workspace_bytes, stream)


def fp8_counters_reset(ctr, stream) -> int:
    return lib().fp8_counters_reset(ctr, stream)


# ---------------------------------------------------------------- torch-level helpers
def _torch():
    import torch
    return torch


def _stream():
    """The current HIP stream of the current device, as an integer handle.
    torch's raw-stream query is used when it exists (it skips building a
    Stream object, about 3 us per call on the host)."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError("inputs are bfloat16 or float32 tensors")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _ld(t):
    """Leading dimension of a 2-D tensor (an empty tensor's stride may be 0)."""
    return t.stride(0) if t.shape[0] > 0 else max(t.shape[1], 1)


# Host-side checks of every tensor handed to the C ABI.  The library sees raw
# device pointers and cannot tell an undersized, mistyped or host-resident
# buffer from a good one, so the binding checks dtype, shape, strides and
# device before anything is enqueued, and raises ValueError on a mismatch.
# Shape and dtype checks come first; the device check (CUDA, one device for
# all tensors of a call) last.
def _check_tensor(t, name, dtypes, shape=None, contiguous=False, unit_col_stride=False):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if unit_col_stride and (t.dim() != 2 or (t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1)):
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")


def _check_scale(t, name, gran, rows, cols):
    torch = _torch()
    want = scale_shape(gran, rows, cols)
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be torch.float32, got {t.dtype}")
    if not t.is_contiguous() or t.numel() != int(_prod(want)):
        raise ValueError(f"{name} must be a contiguous float32 tensor of {int(_prod(want))} elements "
                         f"(shape {want} for this granularity), got shape {tuple(t.shape)}")


def _prod(shape):
    n = 1
    for d in shape:
        n *= int(d)
    return n


def _check_devices(*tensors):
    """Every tensor given is on one CUDA device."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"tensors must be on a CUDA (HIP) device, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors of one call must share a device ({dev} vs {t.device})")


def scale_shape(gran: int, rows: int, cols: int) -> tuple[int, ...]:
    nt = -(-cols // 128)
    if gran == TENSOR:
        return (1,)
    if gran in (ROW_1x128, ROW_1x128_POW2):
        return (rows, nt)
    return (-(-rows // 128), nt)


class Counters:
    """The 4 x uint64 telemetry block in device memory (saturated, underflow,
    nan, nonfinite_out)."""
    FIELDS = ("saturated", "underflow", "nan", "nonfinite_out")

    def __init__(self, device="cuda"):
        torch = _torch()
        self.buf = torch.zeros(4, dtype=torch.int64, device=device)

    def ptr(self):
        return self.buf.data_ptr()

    def reset(self):
        check(fp8_counters_reset(self.ptr(), _stream()))

    def read(self) -> dict:
        vals = self.buf.cpu().tolist()
        return {f: int(v) & 0xFFFFFFFFFFFFFFFF for f, v in zip(self.FIELDS, vals)}


def amax(x, gran: int = TENSOR, workspace=None):
    """workspace: optional uint8 device tensor of at least
    fp8_amax_workspace_size(rows, cols, gran) bytes (allocated per call when
    None)."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16, torch.float32), unit_col_stride=True)
    if workspace is not None:
        _check_tensor(workspace, "workspace", (torch.uint8,), contiguous=True)
    _check_devices(x, workspace)
    rows, cols = x.shape
    out = torch.empty(scale_shape(gran, rows, cols), dtype=torch.float32, device=x.device)
    wsb = lib().fp8_amax_workspace_size(rows, cols, gran)
    if workspace is not None and workspace.numel() < wsb:
        raise ValueError(f"workspace needs {wsb} bytes, got {workspace.numel()}")
    ws = workspace if workspace is not None else torch.empty(max(wsb, 1), dtype=torch.uint8, device=x.device)
    check(fp8_amax(x.data_ptr(), _dtype_code(x), rows, cols, x.stride(0), gran, out.data_ptr(),
                   ws.data_ptr(), ws.numel(), _stream()))
    return out


def quantize(x, fmt: int = E4M3, gran: int = TENSOR, mode: int = FROM_AMAX, scale=None,
             want_t: bool = False, counters: Counters | None = None, out=None, out_t=None, workspace=None):
    """Returns (q uint8 [rows, cols], q_t uint8 [cols, rows] or None, scale fp32).
    workspace: optional uint8 device tensor of at least
    fp8_quantize_workspace_size(rows, cols, gran, mode) bytes (allocated per
    call when not given)."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16, torch.float32), unit_col_stride=True)
    rows, cols = x.shape
    if scale is None:
        if mode == GIVEN:
            raise ValueError("GIVEN mode needs a scale tensor")
    else:
        _check_scale(scale, "scale", gran, rows, cols)
    if out is not None:
        _check_tensor(out, "out", (torch.uint8,), (rows, cols), unit_col_stride=True)
    if want_t and out_t is not None:
        _check_tensor(out_t, "out_t", (torch.uint8,), (cols, rows), unit_col_stride=True)
    if out_t is not None and not want_t:
        raise ValueError("out_t given without want_t=True")
    if workspace is not None:
        _check_tensor(workspace, "workspace", (torch.uint8,), contiguous=True)
    _check_devices(x, scale, out, out_t, workspace, counters.buf if counters else None)
    wsb = lib().fp8_quantize_workspace_size(rows, cols, gran, mode)
    if workspace is not None and workspace.numel() < wsb:
        raise ValueError(f"workspace needs {wsb} bytes, got {workspace.numel()}")
    if scale is None:
        scale = torch.empty(scale_shape(gran, rows, cols), dtype=torch.float32, device=x.device)
    q = out if out is not None else torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qt = None
    if want_t:
        qt = out_t if out_t is not None else torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    ws = workspace if workspace is not None else torch.empty(max(wsb, 1), dtype=torch.uint8, device=x.device)
    check(fp8_quantize(x.data_ptr(), _dtype_code(x), rows, cols, _ld(x), fmt, gran, mode,
                       scale.data_ptr(), q.data_ptr(), _ld(q),
                       _ptr(qt), _ld(qt) if qt is not None else 0,
                       counters.ptr() if counters else None, ws.data_ptr(), ws.numel(), _stream()))
    return q, qt, scale


class AmaxHistory:
    """Device state of delayed scaling for one tensor: the amax of its last
    `length` quantizations (float32, zeros at the start) and the slot of the
    oldest entry (int32)."""

    def __init__(self, length: int = 16, device="cuda"):
        torch = _torch()
        self.length = int(length)
        self.values = torch.zeros(self.length, dtype=torch.float32, device=device)
        self.pos = torch.zeros(1, dtype=torch.int32, device=device)


def quantize_delayed(x, fmt: int, history: AmaxHistory, scale=None, want_t: bool = False,
                     counters: Counters | None = None, out=None, out_t=None, workspace=None):
    """Per-tensor quantize with the scale of the recorded amax history, then
    record this tensor's amax.  Returns (q, q_t or None, scale)."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16, torch.float32), unit_col_stride=True)
    rows, cols = x.shape
    if scale is not None:
        _check_scale(scale, "scale", TENSOR, rows, cols)
    if out is not None:
        _check_tensor(out, "out", (torch.uint8,), (rows, cols), unit_col_stride=True)
    if want_t and out_t is not None:
        _check_tensor(out_t, "out_t", (torch.uint8,), (cols, rows), unit_col_stride=True)
    if out_t is not None and not want_t:
        raise ValueError("out_t given without want_t=True")
    _check_tensor(history.values, "history.values", (torch.float32,), (history.length,), contiguous=True)
    _check_tensor(history.pos, "history.pos", (torch.int32,), (1,), contiguous=True)
    if workspace is not None:
        _check_tensor(workspace, "workspace", (torch.uint8,), contiguous=True)
    _check_devices(x, scale, out, out_t, history.values, history.pos, workspace,
                   counters.buf if counters else None)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    q = out if out is not None else torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qt = None
    if want_t:
        qt = out_t if out_t is not None else torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    wsb = lib().fp8_quantize_delayed_workspace_size(rows, cols)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    check(fp8_quantize_delayed(x.data_ptr(), _dtype_code(x), rows, cols, x.stride(0), fmt,
                               history.values.data_ptr(), history.pos.data_ptr(), history.length,
                               scale.data_ptr(), q.data_ptr(), q.stride(0),
                               _ptr(qt), qt.stride(0) if qt is not None else 0,
                               counters.ptr() if counters else None, workspace.data_ptr(), workspace.numel(),
                               _stream()))
    return q, qt, scale


def scaled_mm(a, fa: int, scale_a, ga: int, b, fb: int, scale_b, gb: int,
              out=None, counters: Counters | None = None, workspace=None):
    """y = (s_a A)(s_b B)^T, a [m,k] uint8, b [n,k] uint8 -> bf16 [m,n]."""
    torch = _torch()
    _check_tensor(a, "a", (torch.uint8,), unit_col_stride=True)
    _check_tensor(b, "b", (torch.uint8,), unit_col_stride=True)
    m, k = a.shape
    n, k2 = b.shape
    if k != k2:
        raise ValueError("a and b disagree on k")
    if ga not in (TENSOR, ROW_1x128, ROW_1x128_POW2) or gb not in (TENSOR, BLOCK_128x128, BLOCK_128x128_POW2):
        raise ValueError("scale_a is TENSOR or ROW_1x128(_POW2), scale_b TENSOR or BLOCK_128x128(_POW2)")
    _check_scale(scale_a, "scale_a", ga, m, k)
    _check_scale(scale_b, "scale_b", gb, n, k)
    if out is not None:
        _check_tensor(out, "out", (torch.bfloat16,), (m, n), unit_col_stride=True)
    if workspace is not None:
        _check_tensor(workspace, "workspace", (torch.uint8,), contiguous=True)
    _check_devices(a, b, scale_a, scale_b, out, workspace, counters.buf if counters else None)
    c = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    wsb = lib().fp8_scaled_mm_workspace_size(m, n, k, ga, gb)
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=a.device)
    check(fp8_scaled_mm(a.data_ptr(), fa, _ld(a), scale_a.data_ptr(), ga,
                        b.data_ptr(), fb, _ld(b), scale_b.data_ptr(), gb,
                        m, n, k, c.data_ptr(), _ld(c),
                        _ptr(workspace), workspace.numel() if workspace is not None else 0,
                        counters.ptr() if counters else None, _stream()))
    return c


def quantize_scaled_mm(x, fa: int, b, fb: int, scale_b, out=None, want_q: bool = False, want_t: bool = False,
                       counters: Counters | None = None, scale_a=None, out_q=None, out_t=None, workspace=None):
    """The forward projection with its bf16 activation quantized on the way
    in: y = bf16(s_a s_b (Q(x) B^T)) with s_a the per-tensor amax scale of x.
    x bf16 [m, 768], b uint8 [n, 768].  Returns (y, scale_a, xq or None,
    xq_t or None); the codes equal those of quantize(x, fa, TENSOR)."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16,), unit_col_stride=True)
    _check_tensor(b, "b", (torch.uint8,), unit_col_stride=True)
    m, k = x.shape
    n, k2 = b.shape
    if k != k2:
        raise ValueError("x and b disagree on k")
    _check_scale(scale_b, "scale_b", TENSOR, n, k)
    if scale_a is not None:
        _check_scale(scale_a, "scale_a", TENSOR, m, k)
    if out is not None:
        _check_tensor(out, "out", (torch.bfloat16,), (m, n), unit_col_stride=True)
    if out_q is not None:
        _check_tensor(out_q, "out_q", (torch.uint8,), (m, k), unit_col_stride=True)
    if out_t is not None:
        _check_tensor(out_t, "out_t", (torch.uint8,), (k, m), unit_col_stride=True)
    if workspace is not None:
        _check_tensor(workspace, "workspace", (torch.uint8,), contiguous=True)
    _check_devices(x, b, scale_b, scale_a, out, out_q, out_t, workspace, counters.buf if counters else None)
    c = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    sa = scale_a if scale_a is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    xq = out_q if out_q is not None else (torch.empty((m, k), dtype=torch.uint8, device=x.device) if want_q else None)
    xqt = out_t if out_t is not None else (torch.empty((k, m), dtype=torch.uint8, device=x.device) if want_t else None)
    wsb = lib().fp8_quantize_scaled_mm_workspace_size(m, n, k)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    check(fp8_quantize_scaled_mm(x.data_ptr(), _ld(x), fa, sa.data_ptr(),
                                 _ptr(xq), _ld(xq) if xq is not None else 0,
                                 _ptr(xqt), _ld(xqt) if xqt is not None else 0,
                                 b.data_ptr(), fb, _ld(b), scale_b.data_ptr(), m, n, k,
                                 c.data_ptr(), _ld(c), counters.ptr() if counters else None,
                                 workspace.data_ptr(), workspace.numel(), _stream()))
    return c, sa, xq, xqt


class WeightCache:
    """FP8 compute copy of one master weight [rows, cols] ("#84 FP8
    Precision", section "Hardware precision": re-quantized after each optimizer
    step, read by the next forward).  q is the [N, K] operand of the forward
    GEMM, q_t the K-contiguous operand of the backward dX GEMM."""

    def __init__(self, rows: int, cols: int, fmt: int = E4M3, gran: int = TENSOR,
                 with_t: bool = True, counters: Counters | None = None, device="cuda"):
        torch = _torch()
        self.rows, self.cols, self.fmt, self.gran = rows, cols, fmt, gran
        self.q = torch.empty((rows, cols), dtype=torch.uint8, device=device)
        self.q_t = torch.empty((cols, rows), dtype=torch.uint8, device=device) if with_t else None
        self.scale = torch.empty(scale_shape(gran, rows, cols), dtype=torch.float32, device=device)
        self.counters = counters

    def desc(self) -> WeightCacheDesc:
        return WeightCacheDesc(self.rows, self.cols, self.fmt, self.gran, self.q.data_ptr(),
                               _ptr(self.q_t), self.scale.data_ptr(),
                               self.counters.ptr() if self.counters else None)


class RequantPlan:
    """A prepared refresh of a fixed list of caches from a fixed list of
    masters: the argument checks, the descriptor array and the workspace are
    set up once, and each call is one C call (the refresh after every
    optimizer step of a training loop).  The masters and caches are held by
    reference; their storage must stay where it is."""

    def __init__(self, caches: list[WeightCache], masters: list):
        torch = _torch()
        if len(caches) != len(masters):
            raise ValueError("one master per cache")
        for c, m in zip(caches, masters):
            _check_tensor(m, "master", (torch.bfloat16, torch.float32), (c.rows, c.cols), contiguous=True)
        if caches:
            _check_devices(*masters, *[c.q for c in caches])
        self.caches, self.masters = list(caches), list(masters)
        n = len(caches)
        self._n = n
        self._descs = (WeightCacheDesc * max(n, 1))(*[c.desc() for c in caches])
        self._masters = (ctypes.c_void_p * max(n, 1))(*[m.data_ptr() for m in masters])
        self._dtypes = (ctypes.c_int * max(n, 1))(*[_dtype_code(m) for m in masters])
        self._wsb = lib().fp8_requant_workspace_size(self._descs, n) if n else 0
        self._ws = torch.empty(max(self._wsb, 1), dtype=torch.uint8,
                               device=masters[0].device if n else "cpu")

    def __call__(self) -> None:
        if self._n:
            check(lib().fp8_requant_weights(self._descs, self._masters, self._dtypes, self._n,
                                            self._ws.data_ptr(), self._wsb, _stream()))


def requant_weights(caches: list[WeightCache], masters: list) -> None:
    """Refresh every cache from its master in one call."""
    if not caches:
        return
    RequantPlan(caches, masters)()
