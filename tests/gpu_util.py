"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm
import oracle

FMT_NAME = {fm.E4M3: "e4m3", fm.E5M2: "e5m2"}
THREADS = min(16, os.cpu_count() or 1)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fm.load()  # raises if the library is missing: no fallback


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def codes(t: torch.Tensor, rows: int, cols: int) -> np.ndarray:
    return host(t)[:rows, :cols]


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, np.float32)).view(np.uint32)


def same_f32(a, b) -> bool:
    """Bitwise equality, except that any NaN matches any NaN."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and np.array_equal(f32_bits(a)[~na], f32_bits(b)[~nb]))


def acc_amax(acc: torch.Tensor) -> np.float32:
    """The amax a delayed-scaling accumulator holds: its largest slot, compared
    as |x| bit patterns so that a NaN slot wins."""
    bits = host(acc).view(np.uint32)
    return np.uint32(bits.max()).view(np.float32)


def parallel_encode(fmt: str, v: np.ndarray) -> np.ndarray:
    """oracle.encode over a large array, split across threads (ctypes drops the GIL)."""
    oracle.encode(fmt, np.zeros(1, np.float32))  # build the oracle's table once
    out = np.empty(v.shape, np.uint8)
    parts = np.array_split(np.arange(v.size), THREADS)

    def work(idx):
        if idx.size:
            out.reshape(-1)[idx[0]:idx[-1] + 1] = oracle.encode(fmt, v.reshape(-1)[idx[0]:idx[-1] + 1])

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(work, parts))
    return out


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def padded_codes(q: np.ndarray) -> torch.Tensor:
    """Upload codes [R x C] into a [R x ceil16(C)] device buffer (16-byte rows)."""
    r, c = q.shape
    ld = max(16, (c + 15) // 16 * 16)
    buf = np.zeros((r, ld), np.uint8)
    buf[:, :c] = q
    return dev(buf)
