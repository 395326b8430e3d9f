"""Binding of libfp8mi_probe.so (include/fp8mi_probe.h): the measurement
kernels bench.py uses to state what this GPU sustains -- the FP8 matrix-core
rate and shader clock under full load (fixed and varied operands), HBM
streams at the quantize
kernels' read:write mixes, and the cost of an empty launch.  Argument
marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8mi_probe.so")

READ, COPY, HALF, SPLIT = 0, 1, 2, 3
NT_LOAD, NT_STORE, BLOCKED = 16, 32, 64  # access hints, OR-ed into a mix
EXPORTS = ("fp8probe_stream", "fp8probe_mfma", "fp8probe_mfma_varied", "fp8probe_empty", "fp8probe_wall_clock_khz")
MFMA_WAVES = 8                  # waves per workgroup of fp8probe_mfma
MFMA_FLOPS_PER_ROUND = 8 * 2 * 16 * 16 * 128  # eight 16x16x128 products per wave per round

_lib = None


def load(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not built; run python -m fp8_scaled_quantization_scale_amd.build")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.fp8probe_stream.restype = i32
    lib.fp8probe_stream.argtypes = [vp, i64, vp, vp, i32, vp]
    lib.fp8probe_mfma.restype = i32
    lib.fp8probe_mfma.argtypes = [i32, i32, vp, vp, vp]
    lib.fp8probe_mfma_varied.restype = i32
    lib.fp8probe_mfma_varied.argtypes = [i32, i32, vp, vp, vp]
    lib.fp8probe_empty.restype = i32
    lib.fp8probe_empty.argtypes = [i32, i32, vp]
    lib.fp8probe_wall_clock_khz.restype = i32
    lib.fp8probe_wall_clock_khz.argtypes = [vp]
    _lib = lib
    return lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def stream(src: torch.Tensor, dst0: torch.Tensor, dst1: torch.Tensor | None, mix: int) -> None:
    """One pass of fp8probe_stream over all of src (contiguous device tensors;
    dst sizes as the header states: checked here).  mix may carry NT_LOAD,
    NT_STORE and BLOCKED."""
    n16 = src.numel() * src.element_size() // 16
    base = mix & 15
    out = n16 if base == COPY else (n16 // 2 if base in (HALF, SPLIT) else 1)
    for t in (src, dst0) + ((dst1,) if base == SPLIT else ()):
        if not (t.is_cuda and t.is_contiguous()):
            raise RuntimeError("probe buffers must be contiguous device tensors")
    if dst0.numel() * dst0.element_size() < 16 * out or (base == SPLIT and dst1.numel() * dst1.element_size() < 16 * out):
        raise RuntimeError("probe output buffer too small")
    st = load().fp8probe_stream(src.data_ptr(), n16, dst0.data_ptr(), None if dst1 is None else dst1.data_ptr(),
                                mix, _stream())
    if st != 0:
        raise RuntimeError(f"fp8probe_stream failed ({st})")


def mfma(iters: int, workgroups: int, clocks: torch.Tensor, sink: torch.Tensor, varied: bool = False) -> None:
    """One launch of fp8probe_mfma (fixed operands) or, with varied=True,
    fp8probe_mfma_varied (operands that change from product to product);
    clocks: int64 [4 * workgroups], sink: float32 [1], both on the device."""
    for t in (clocks, sink):
        if not (t.is_cuda and t.is_contiguous()):
            raise RuntimeError("probe buffers must be contiguous device tensors")
    if clocks.numel() < 4 * workgroups or clocks.dtype != torch.int64 or sink.dtype != torch.float32:
        raise RuntimeError("clocks must be int64 [4 * workgroups], sink float32")
    fn = load().fp8probe_mfma_varied if varied else load().fp8probe_mfma
    st = fn(iters, workgroups, clocks.data_ptr(), sink.data_ptr(), _stream())
    if st != 0:
        raise RuntimeError(f"fp8probe_mfma{'_varied' if varied else ''} failed ({st})")


def empty(workgroups: int = 1, threads: int = 256) -> None:
    """One launch of fp8probe_empty (a kernel that does nothing)."""
    st = load().fp8probe_empty(workgroups, threads, _stream())
    if st != 0:
        raise RuntimeError(f"fp8probe_empty failed ({st})")


def wall_clock_khz() -> int:
    """Rate of the wall counter fp8probe_mfma records (kHz)."""
    khz = load().fp8probe_wall_clock_khz(_stream())
    if khz <= 0:
        raise RuntimeError("fp8probe_wall_clock_khz failed")
    return khz
