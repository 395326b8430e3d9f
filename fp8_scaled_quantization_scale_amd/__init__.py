"""Python binding of libfp8mi.so, the MI355X (gfx950) FP8 scaled-quantization
and scaled-FP8-GEMM library.

The three entry points keep the C names and arguments of include/fp8mi.h
(``fp8_quantize``, ``fp8_amax_history_update``, ``fp8_gemm_scaled``); this
module only marshals torch tensors into device pointers and passes torch's
current HIP stream.  Every step of the computation runs in the library's
kernels.  ``quantize`` / ``gemm`` / ``DelayedState`` below allocate the output
tensors with torch and call those same entry points.

Importing this module does not load the library; the first call does, and
raises if it has not been built (``python -m fp8_scaled_quantization_scale_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8mi.so")

# values of the FP8MI_* macros in include/fp8mi.h
OK = 0
ERR_NULL, ERR_ENUM, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_HIP = -1, -2, -3, -4, -5, -6
E4M3, E5M2 = 0, 1
IN_BF16, IN_FP32 = 0, 1
OUT_BF16, OUT_FP32 = 0, 1
TENSOR_CURRENT, TENSOR_DELAYED, BLOCK_1x128, BLOCK_128x128, MX_1x32 = 0, 1, 2, 3, 4
CHANNEL, MX_1x32_OCP = 5, 6
ROW, COL, ROW_AND_COL = 1, 2, 3
GEMM_TENSOR, GEMM_BLOCK_1x128_128x128, GEMM_BLOCK_1x128_1x128, GEMM_MX_1x32 = 0, 1, 2, 3
GEMM_BLOCK_128x128_128x128, GEMM_CHANNEL = 4, 5
LAYOUT_TN = 0
AMAX_SLOTS = 1024  # floats in the amax array of a per-tensor cast

FMT = {"e4m3": E4M3, "e5m2": E5M2}
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}

EXPORTS = ("fp8_quantize", "fp8_quantize_static_scratch", "fp8_amax_history_update", "fp8_gemm_scaled",
           "fp8_bf16_gemm", "fp8_status_string", "fp8_version")


class Fp8Error(RuntimeError):
    pass


_lib = None


def load(path: str = LIB_PATH):
    """Load libfp8mi.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise Fp8Error(f"{path} not built; run python -m fp8_scaled_quantization_scale_amd.build")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.fp8_quantize.restype = i32
    lib.fp8_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, i32, i32,
                                 vp, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp]
    lib.fp8_quantize_static_scratch.restype = i32
    lib.fp8_quantize_static_scratch.argtypes = lib.fp8_quantize.argtypes
    lib.fp8_amax_history_update.restype = i32
    lib.fp8_amax_history_update.argtypes = [vp, vp, i64, vp, i32, i32, vp, vp, vp, vp]
    lib.fp8_gemm_scaled.restype = i32
    lib.fp8_gemm_scaled.argtypes = [vp, i32, vp, i64, vp, i32, vp, i64, i32, i32, i64, i64, i64,
                                    vp, i32, i64, vp]
    lib.fp8_bf16_gemm.restype = i32
    lib.fp8_bf16_gemm.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, i32, i64, vp]
    lib.fp8_status_string.restype = ctypes.c_char_p
    lib.fp8_status_string.argtypes = [i32]
    lib.fp8_version.restype = i32
    lib.fp8_version.argtypes = []
    _lib = lib
    return lib


def _p(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise Fp8Error("tensor arguments must be device tensors (the kernels read and write them on the GPU)")
    return t.data_ptr()


def _need(ok: bool, msg: str):
    if not ok:
        raise Fp8Error(msg)


def _matrix(name: str, t, dtypes) -> None:
    """A 2-D device tensor with unit column stride and one of `dtypes`."""
    _need(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a device tensor")
    _need(t.dim() == 2 and t.stride(1) == 1, f"{name} must be 2-D with unit column stride")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}; expected one of {dtypes}")


def _vector(name: str, t, dtype, n: int) -> None:
    """A contiguous device tensor of `dtype` holding at least `n` elements."""
    _need(isinstance(t, torch.Tensor) and t.is_cuda, f"{name} must be a device tensor")
    _need(t.dtype == dtype, f"{name} has dtype {t.dtype}; expected {dtype}")
    _need(t.is_contiguous() and t.numel() >= n, f"{name} must be contiguous with at least {n} elements")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != OK:
        msg = load().fp8_status_string(status).decode()
        raise Fp8Error(f"{what} failed ({status}): {msg}")


def status_string(status: int) -> str:
    return load().fp8_status_string(status).decode()


def version() -> int:
    return load().fp8_version()


# ---------------------------------------------------------------------------
# the C entry points, argument for argument (tensors or raw pointers)
# ---------------------------------------------------------------------------

def fp8_quantize(x, x_dtype, rows, cols, ld_x, recipe, fmt, orient, margin,
                 q_row, ld_q_row, s_row, q_col, ld_q_col, s_col,
                 scale, scale_inv, amax, nonfinite, stream=None) -> int:
    return load().fp8_quantize(_p(x), x_dtype, rows, cols, ld_x, recipe, fmt, orient, margin,
                               _p(q_row), ld_q_row, _p(s_row), _p(q_col), ld_q_col, _p(s_col),
                               _p(scale), _p(scale_inv), _p(amax), _p(nonfinite), _stream(stream))


def fp8_quantize_static_scratch(x, x_dtype, rows, cols, ld_x, recipe, fmt, orient, margin,
                                q_row, ld_q_row, s_row, q_col, ld_q_col, s_col,
                                scale, scale_inv, amax, nonfinite, stream=None) -> int:
    """fp8_quantize with current scaling's partial maxima in the library's
    static device scratch (amax: one float for TENSOR_CURRENT)."""
    return load().fp8_quantize_static_scratch(_p(x), x_dtype, rows, cols, ld_x, recipe, fmt, orient, margin,
                                              _p(q_row), ld_q_row, _p(s_row), _p(q_col), ld_q_col, _p(s_col),
                                              _p(scale), _p(scale_inv), _p(amax), _p(nonfinite), _stream(stream))


def fp8_amax_history_update(history, head, length, amax, fmt, margin, scale, scale_inv,
                            nonfinite, stream=None) -> int:
    return load().fp8_amax_history_update(_p(history), _p(head), length, _p(amax), fmt, margin,
                                          _p(scale), _p(scale_inv), _p(nonfinite), _stream(stream))


def fp8_gemm_scaled(a, fmt_a, s_a, lda, b, fmt_b, s_b, ldb, recipe, layout, M, N, K, c, c_dtype, ldc,
                    stream=None) -> int:
    return load().fp8_gemm_scaled(_p(a), fmt_a, _p(s_a), lda, _p(b), fmt_b, _p(s_b), ldb, recipe, layout,
                                  M, N, K, _p(c), c_dtype, ldc, _stream(stream))


def fp8_bf16_gemm(a, lda, b, ldb, M, N, K, c, c_dtype, ldc, stream=None) -> int:
    return load().fp8_bf16_gemm(_p(a), lda, _p(b), ldb, M, N, K, _p(c), c_dtype, ldc, _stream(stream))


# ---------------------------------------------------------------------------
# conveniences: allocate outputs with torch, call the entry points above
# ---------------------------------------------------------------------------

def _ceil(a: int, b: int) -> int:
    return (a + b - 1) // b


def _pad16(n: int) -> int:
    return _ceil(max(n, 1), 16) * 16


@dataclass
class Quantized:
    """Codes (uint8) and scales of one fp8_quantize call."""
    fmt: int
    recipe: int
    q_row: torch.Tensor | None = None   # [rows x ld_q_row] codes, first `cols` columns used
    s_row: torch.Tensor | None = None
    q_col: torch.Tensor | None = None   # [cols x ld_q_col] codes of x^T
    s_col: torch.Tensor | None = None
    scale: torch.Tensor | None = None
    scale_inv: torch.Tensor | None = None
    amax: torch.Tensor | None = None
    nonfinite: torch.Tensor | None = None


def scale_grid_shape(recipe: int, rows: int, cols: int, orient: int):
    """Shape and dtype of the ROW (orient=ROW) or COL scale grid of fp8_quantize."""
    if recipe == BLOCK_1x128:
        return ((rows, _ceil(cols, 128)) if orient == ROW else (cols, _ceil(rows, 128))), torch.float32
    if recipe == BLOCK_128x128:
        g = (_ceil(rows, 128), _ceil(cols, 128))
        return (g if orient == ROW else (g[1], g[0])), torch.float32
    if recipe in (MX_1x32, MX_1x32_OCP):
        return ((rows, _ceil(cols, 32)) if orient == ROW else (cols, _ceil(rows, 32))), torch.uint8
    if recipe == CHANNEL:
        return ((rows,) if orient == ROW else (cols,)), torch.float32
    return None, None


def quantize(x: torch.Tensor, recipe: int, fmt: int, orient: int = ROW, margin: int = 0,
             scale: torch.Tensor | None = None, amax: torch.Tensor | None = None,
             nonfinite: torch.Tensor | None = None, stream=None) -> Quantized:
    """Quantize a 2-D BF16/FP32 device tensor (row-major, ld = its stride)."""
    _matrix("x", x, (torch.bfloat16, torch.float32))
    if scale is not None:
        _vector("scale", scale, torch.float32, 1)
    if amax is not None:
        _need(isinstance(amax, torch.Tensor) and amax.is_cuda and amax.dtype == torch.float32
              and amax.is_contiguous(), "amax must be a contiguous float32 device tensor")
    if nonfinite is not None:
        _vector("nonfinite", nonfinite, torch.int32, 1)
    rows, cols = x.shape
    dev = x.device
    x_dtype = IN_BF16 if x.dtype == torch.bfloat16 else IN_FP32
    out = Quantized(fmt=fmt, recipe=recipe)
    ld_r = _pad16(cols)
    ld_c = _pad16(rows)
    if orient & ROW:
        out.q_row = torch.empty(rows, ld_r, dtype=torch.uint8, device=dev)
        shp, dt = scale_grid_shape(recipe, rows, cols, ROW)
        if shp is not None:
            out.s_row = torch.empty(shp, dtype=dt, device=dev)
    if orient & COL:
        out.q_col = torch.empty(cols, ld_c, dtype=torch.uint8, device=dev)
        shp, dt = scale_grid_shape(recipe, rows, cols, COL)
        if shp is not None:
            out.s_col = torch.empty(shp, dtype=dt, device=dev)
    if recipe in (TENSOR_CURRENT, TENSOR_DELAYED):
        out.scale = scale if scale is not None else torch.ones(1, dtype=torch.float32, device=dev)
        if recipe == TENSOR_CURRENT:  # delayed leaves scale_inv to the history update
            out.scale_inv = torch.empty(1, dtype=torch.float32, device=dev)
        if amax is None:
            amax = torch.zeros(AMAX_SLOTS, dtype=torch.float32, device=dev)
        if amax.numel() < AMAX_SLOTS:
            raise Fp8Error(f"the amax array of a per-tensor cast holds {AMAX_SLOTS} floats")
        out.amax = amax
    out.nonfinite = nonfinite
    st = fp8_quantize(x, x_dtype, rows, cols, x.stride(0), recipe, fmt, orient, margin,
                      out.q_row, ld_r, out.s_row, out.q_col, ld_c, out.s_col,
                      out.scale, out.scale_inv, out.amax, nonfinite, stream)
    _check(st, "fp8_quantize")
    return out


_OUT_DTYPES = {torch.bfloat16: OUT_BF16, torch.float32: OUT_FP32}


def _scale_need(recipe: int, rows: int, K: int, is_a: bool):
    """(elements, dtype) of the scale grid fp8_gemm_scaled reads for one
    operand with `rows` rows (M for a, N for b) and contraction K."""
    kb = _ceil(K, 128)
    if recipe == GEMM_TENSOR:
        return 1, torch.float32
    if recipe == GEMM_CHANNEL:
        return rows, torch.float32
    if recipe == GEMM_MX_1x32:
        return rows * _ceil(K, 32), torch.uint8
    if recipe == GEMM_BLOCK_128x128_128x128 or (recipe == GEMM_BLOCK_1x128_128x128 and not is_a):
        return _ceil(rows, 128) * kb, torch.float32
    if recipe in (GEMM_BLOCK_1x128_128x128, GEMM_BLOCK_1x128_1x128):
        return rows * kb, torch.float32
    raise Fp8Error(f"unknown GEMM recipe {recipe}")


def gemm(a: torch.Tensor, fmt_a: int, s_a: torch.Tensor, b: torch.Tensor, fmt_b: int,
         s_b: torch.Tensor, recipe: int, K: int, out_dtype=torch.bfloat16,
         M: int | None = None, N: int | None = None, c: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """C[M x N] = dequant(a[:, :K]) . dequant(b[:, :K])^T (a, b uint8 codes, row-major).

    Checks every tensor against the sizes the kernels will touch (the C entry
    point takes plain pointers and cannot), so a wrong size is an Fp8Error
    here rather than an out-of-bounds access on the GPU."""
    codes = (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2)
    _matrix("a", a, codes)
    _matrix("b", b, codes)
    M = a.shape[0] if M is None else M
    N = b.shape[0] if N is None else N
    _need(M >= 0 and N >= 0 and K >= 0, "M, N, K must be non-negative")
    if c is None:
        _need(out_dtype in _OUT_DTYPES, f"out_dtype must be one of {tuple(_OUT_DTYPES)}")
        c = torch.empty(M, N, dtype=out_dtype, device=a.device)
    _matrix("c", c, tuple(_OUT_DTYPES))
    _need(c.shape[0] >= M and c.shape[1] >= N, f"c is {tuple(c.shape)}; needs at least {M} x {N}")
    if M > 0 and N > 0 and K > 0:
        _need(a.shape[0] >= M and a.shape[1] >= K, f"a is {tuple(a.shape)}; needs at least {M} x {K}")
        _need(b.shape[0] >= N and b.shape[1] >= K, f"b is {tuple(b.shape)}; needs at least {N} x {K}")
        for name, t, (n, dt) in (("s_a", s_a, _scale_need(recipe, M, K, True)),
                                 ("s_b", s_b, _scale_need(recipe, N, K, False))):
            _vector(name, t, dt, n)
    c_dtype = _OUT_DTYPES[c.dtype]
    st = fp8_gemm_scaled(a, fmt_a, s_a, a.stride(0), b, fmt_b, s_b, b.stride(0), recipe, LAYOUT_TN,
                         M, N, K, c, c_dtype, c.stride(0), stream)
    _check(st, "fp8_gemm_scaled")
    return c


def bf16_gemm(a: torch.Tensor, b: torch.Tensor, out_dtype=torch.bfloat16,
              c: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """C[M x N] = a[M x K] . b[N x K]^T, BF16 operands (row-major, unit column stride)."""
    _matrix("a", a, (torch.bfloat16,))
    _matrix("b", b, (torch.bfloat16,))
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] >= K, f"b is {tuple(b.shape)}; needs at least {N} x {K}")
    if c is None:
        _need(out_dtype in _OUT_DTYPES, f"out_dtype must be one of {tuple(_OUT_DTYPES)}")
        c = torch.empty(M, N, dtype=out_dtype, device=a.device)
    _matrix("c", c, tuple(_OUT_DTYPES))
    _need(c.shape[0] >= M and c.shape[1] >= N, f"c is {tuple(c.shape)}; needs at least {M} x {N}")
    c_dtype = _OUT_DTYPES[c.dtype]
    _check(fp8_bf16_gemm(a, a.stride(0), b, b.stride(0), M, N, K, c, c_dtype, c.stride(0), stream),
           "fp8_bf16_gemm")
    return c


class DelayedState:
    """Device-resident delayed-scaling state: amax ring, head, scale,
    scale_inv, the amax accumulator (AMAX_SLOTS per-workgroup slots, folded
    by the history update) and a non-finite counter."""

    def __init__(self, fmt: int, length: int = 200, margin: int = 0, device="cuda"):
        self.fmt, self.length, self.margin = fmt, length, margin
        self.history = torch.zeros(length, dtype=torch.float32, device=device)
        self.head = torch.zeros(1, dtype=torch.int32, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(1, dtype=torch.float32, device=device)
        self.amax = torch.zeros(AMAX_SLOTS, dtype=torch.float32, device=device)
        self.nonfinite = torch.zeros(1, dtype=torch.int32, device=device)

    def quantize(self, x: torch.Tensor, orient: int = ROW, stream=None) -> Quantized:
        q = quantize(x, TENSOR_DELAYED, self.fmt, orient, self.margin, scale=self.scale,
                     amax=self.amax, stream=stream)
        q.scale_inv = self.scale_inv.clone()
        return q

    def update(self, stream=None):
        st = fp8_amax_history_update(self.history, self.head, self.length, self.amax, self.fmt,
                                     self.margin, self.scale, self.scale_inv, self.nonfinite, stream)
        _check(st, "fp8_amax_history_update")

    def state_dict(self):
        return {k: getattr(self, k).clone() for k in
                ("history", "head", "scale", "scale_inv", "amax", "nonfinite")}

    def load_state_dict(self, sd):
        for k, v in sd.items():
            getattr(self, k).copy_(v)
