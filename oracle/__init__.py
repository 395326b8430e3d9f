"""CPU oracle for FP8 scaled quantization and scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and never imports it.

The quantization half is plain C (``oracle.c``, loaded through ctypes); the
GEMM half is the textbook definition in float64 numpy: dequantize both
operands with their own scales, then one float64 matrix product.

Sources, cited by page and section:
  [P1] "2025 technical guide: FP8 quantized training" (blog.gitcode.com)
       sec. 2.1-2.3 (recipes), sec. 3.1 (fprop / dgrad / wgrad take
       quantized inputs and keep BF16/FP32 outputs).
  [P3] "Mastering FP8 LLM training" (nmedialink.com), strategies 1-4.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FORMATS = ("e4m3", "e5m2")
_FMT = {"e4m3": 0, "e5m2": 1}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
             "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    vp = ctypes.c_void_p
    lib.or_decode.restype = ctypes.c_double
    lib.or_decode.argtypes = [i32, i32]
    lib.or_encode.restype = i32
    lib.or_encode.argtypes = [i32, f32]
    lib.or_max_value.restype = ctypes.c_double
    lib.or_max_value.argtypes = [i32]
    lib.or_encode_array.argtypes = [i32, vp, vp, i64]
    lib.or_decode_array.argtypes = [i32, vp, vp, i64]
    lib.or_scale_from_amax.restype = i32
    lib.or_scale_from_amax.argtypes = [i32, f32, i32, vp, vp]
    lib.or_amax_block.restype = f32
    lib.or_amax_block.argtypes = [vp, i64, i64, i64, i64, i64]
    lib.or_quantize_current.restype = i32
    lib.or_quantize_current.argtypes = [i32, vp, i64, i64, i32, vp, vp, vp, vp]
    lib.or_quantize_delayed.argtypes = [i32, vp, i64, i64, f32, vp, vp]
    lib.or_quantize_blocks.restype = i64
    lib.or_quantize_blocks.argtypes = [i32, vp, i64, i64, i64, i64, i32, vp, vp]
    lib.or_mx_scale_byte.restype = i32
    lib.or_mx_scale_byte.argtypes = [i32, f32]
    lib.or_e8m0_value.restype = ctypes.c_double
    lib.or_e8m0_value.argtypes = [i32]
    lib.or_quantize_mx.restype = i64
    lib.or_quantize_mx.argtypes = [i32, vp, i64, i64, i64, i64, vp, vp]
    lib.or_mx_scale_byte_floor.restype = i32
    lib.or_mx_scale_byte_floor.argtypes = [i32, f32]
    lib.or_quantize_mx_rule.restype = i64
    lib.or_quantize_mx_rule.argtypes = [i32, vp, i64, i64, i64, i64, i32, vp, vp]
    lib.or_history_update.restype = i32
    lib.or_history_update.argtypes = [vp, vp, i32, f32, i32, i32, vp, vp, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    """Inputs as contiguous float32 (a BF16 tensor widens exactly)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().float().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def decode(fmt: str, codes) -> np.ndarray:
    """float64 value of every code (NaN / +-Inf where the format has them)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    _load().or_decode_array(_FMT[fmt], _ptr(c), _ptr(out), c.size)
    return out


def decode_table(fmt: str) -> np.ndarray:
    return decode(fmt, np.arange(256, dtype=np.uint8))


def max_value(fmt: str) -> float:
    return _load().or_max_value(_FMT[fmt])


def encode(fmt: str, values) -> np.ndarray:
    """Saturating round-to-nearest-even FP8 code of each float32 value."""
    v = _f32(values)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().or_encode_array(_FMT[fmt], _ptr(v), _ptr(out), v.size)
    return out


# ---------------------------------------------------------------------------
# scales and quantization
# ---------------------------------------------------------------------------

def scale_from_amax(fmt: str, amax: float, margin: int = 0):
    """(s, s_inv, nonfinite_flag) for one amax."""
    s = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    flag = _load().or_scale_from_amax(_FMT[fmt], float(np.float32(amax)), margin, _ptr(s), _ptr(si))
    return s[0], si[0], flag


def amax(x) -> np.float32:
    a = _f32(x)
    a2 = a.reshape(1, -1) if a.ndim != 2 else a
    r, c = a2.shape
    return np.float32(_load().or_amax_block(_ptr(a2), c, 0, r, 0, c))


def quantize_current(fmt: str, x, margin: int = 0):
    """Per-tensor current scaling -> (codes, s, s_inv, amax, flag)."""
    a = _f32(x)
    a2 = a.reshape(1, -1) if a.ndim != 2 else a
    r, c = a2.shape
    q = np.empty(a2.shape, np.uint8)
    s = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    am = np.zeros(1, np.float32)
    flag = _load().or_quantize_current(_FMT[fmt], _ptr(a2), r, c, margin, _ptr(q), _ptr(s), _ptr(si), _ptr(am))
    return q.reshape(a.shape), s[0], si[0], am[0], flag


def quantize_delayed(fmt: str, x, s: float):
    """Cast with a carried-over scale -> (codes, amax of this tensor)."""
    a = _f32(x)
    a2 = a.reshape(1, -1) if a.ndim != 2 else a
    r, c = a2.shape
    q = np.empty(a2.shape, np.uint8)
    am = np.zeros(1, np.float32)
    _load().or_quantize_delayed(_FMT[fmt], _ptr(a2), r, c, float(np.float32(s)), _ptr(q), _ptr(am))
    return q.reshape(a.shape), am[0]


def quantize_blocks(fmt: str, x, br: int, bc: int, margin: int = 0):
    """Block scaling with br x bc blocks -> (codes, s_inv grid, n_nonfinite)."""
    a = _f32(x)
    r, c = a.shape
    q = np.empty(a.shape, np.uint8)
    grid = np.empty(((r + br - 1) // br, (c + bc - 1) // bc), np.float32)
    bad = _load().or_quantize_blocks(_FMT[fmt], _ptr(a), r, c, br, bc, margin, _ptr(q), _ptr(grid))
    return q, grid, bad


def mx_scale_byte(fmt: str, amax_value: float, rule: str = "ceil") -> int:
    """E8M0 byte of a block amax: "ceil" = smallest power of two with no
    element saturating; "floor" = the OCP specification's floor(log2 amax) - emax."""
    f = _load().or_mx_scale_byte_floor if rule == "floor" else _load().or_mx_scale_byte
    return f(_FMT[fmt], float(np.float32(amax_value)))


def e8m0_value(byte: int) -> float:
    return _load().or_e8m0_value(int(byte))


def quantize_mx(fmt: str, x, br: int, bc: int, rule: str = "ceil"):
    """MX blocks of br x bc with E8M0 scale bytes -> (codes, bytes, n_nonfinite)."""
    assert rule in ("ceil", "floor")
    a = _f32(x)
    r, c = a.shape
    q = np.empty(a.shape, np.uint8)
    grid = np.empty(((r + br - 1) // br, (c + bc - 1) // bc), np.uint8)
    bad = _load().or_quantize_mx_rule(_FMT[fmt], _ptr(a), r, c, br, bc, int(rule == "floor"),
                                      _ptr(q), _ptr(grid))
    return q, grid, bad


def quantize_channel(fmt: str, x, margin: int = 0):
    """Channel-wise scaling: one scale per row, i.e. block scaling with
    1 x cols blocks -> (codes, s_inv [rows], n_nonfinite).  Per-column
    scales are quantize_channel of the transpose."""
    a = _f32(x)
    q, grid, bad = quantize_blocks(fmt, a, 1, max(a.shape[1], 1), margin)
    return q, grid[:, 0].copy(), bad


class History:
    """Delayed-scaling state: amax ring, head, scale, scale_inv, counter."""

    def __init__(self, fmt: str, length: int = 200, margin: int = 0):
        self.fmt = fmt
        self.length = length
        self.margin = margin
        self.ring = np.zeros(length, np.float32)
        self.head = np.zeros(1, np.int32)
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)
        self.nonfinite = np.zeros(1, np.int32)

    def update(self, amax_value: float) -> int:
        s = np.zeros(1, np.float32)
        si = np.zeros(1, np.float32)
        pushed = _load().or_history_update(
            _ptr(self.ring), _ptr(self.head), self.length, float(np.float32(amax_value)),
            _FMT[self.fmt], self.margin, _ptr(s), _ptr(si), _ptr(self.nonfinite))
        self.scale, self.scale_inv = s[0], si[0]
        return pushed

    def state(self):
        return (self.ring.copy(), int(self.head[0]), np.float32(self.scale),
                np.float32(self.scale_inv), int(self.nonfinite[0]))


# ---------------------------------------------------------------------------
# GEMM reference [P1 sec.3.1]: C = A . B^T over dequantized operands, float64
# ---------------------------------------------------------------------------

def expand_grid(grid: np.ndarray, br: int, bc: int, rows: int, cols: int) -> np.ndarray:
    """Per-element view of a per-block scale grid (blocks br x bc)."""
    g = np.asarray(grid)
    return np.repeat(np.repeat(g, br, axis=0), bc, axis=1)[:rows, :cols]


def dequant(fmt: str, codes, s_inv, br: int | None = None, bc: int | None = None) -> np.ndarray:
    """float64 x = dec(q) * s_inv.  s_inv: a scalar (per-tensor) or a per-block
    grid of float32 values (blocks br x bc)."""
    c = np.asarray(codes, dtype=np.uint8)
    v = decode_table(fmt)[c]
    if br is None:
        return v * float(s_inv)
    return v * expand_grid(np.asarray(s_inv, np.float64), br, bc, *c.shape)


def dequant_mx(fmt: str, codes, scale_bytes, br: int, bc: int) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    v = decode_table(fmt)[c]
    table = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)
    return v * expand_grid(table[np.asarray(scale_bytes, np.uint8)], br, bc, *c.shape)


def gemm_ref(a_deq: np.ndarray, b_deq: np.ndarray):
    """C_ref[i,j] = sum_k a[i,k] b[j,k] and S[i,j] = sum_k |a[i,k] b[j,k]|,
    both float64 (operands stored with the contraction index last)."""
    a = np.asarray(a_deq, np.float64)
    b = np.asarray(b_deq, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        return a @ b.T, np.abs(a) @ np.abs(b).T


def gemm_ref_entries(a_deq: np.ndarray, b_deq: np.ndarray, ii, jj):
    """C_ref and S at the listed (i, j) pairs only."""
    a = np.asarray(a_deq, np.float64)[np.asarray(ii)]
    b = np.asarray(b_deq, np.float64)[np.asarray(jj)]
    with np.errstate(invalid="ignore", over="ignore"):
        return (a * b).sum(axis=1), np.abs(a * b).sum(axis=1)


# Accumulation bound 2^-10 * S; BF16 output adds one output rounding,
# u = 2^-8 of |C_ref|; FP32 output is held to the accumulation bound.
ACC_TOL = 2.0 ** -10
OUT_TOL = {"bf16": 2.0 ** -8, "fp32": 0.0}


def gemm_violations(c, c_ref, s, out: str) -> np.ndarray:
    """Boolean mask of entries outside |C - C_ref| <= 2^-10 S + u_out |C_ref|.
    Non-finite C_ref must be matched by the same class (NaN, +Inf, -Inf)."""
    c = np.asarray(c, np.float64)
    c_ref = np.asarray(c_ref, np.float64)
    s = np.asarray(s, np.float64)
    fin = np.isfinite(c_ref)
    with np.errstate(invalid="ignore"):
        bound = ACC_TOL * s + OUT_TOL[out] * np.abs(c_ref)
        bad_fin = fin & ~(np.abs(c - c_ref) <= bound)
    nan_ref = np.isnan(c_ref)
    inf_ref = np.isinf(c_ref)
    bad_nan = nan_ref & ~np.isnan(c)
    bad_inf = inf_ref & ~(np.isinf(c) & (np.sign(c) == np.sign(c_ref)))
    return bad_fin | bad_nan | bad_inf
