"""fp8_quantize_static_scratch (the entry point for callers that cannot
allocate) against fp8_quantize, through the C ABI: two calls in a row, the
second on a smaller tensor with a smaller amax, so partial maxima the first
call left in the shared static scratch would show in the second call's amax
if they were read.  Codes, scale, scale_inv and amax bit for bit."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm
import workloads
from gpu_util import host, need_gpu, same_f32

pytestmark = pytest.mark.gpu


def _tensor(rows, cols, seed, sigma, dtype):
    return workloads.make(workloads.Tensor("X", rows, cols, "gains", sigma, seed), "cuda").to(dtype)


def _run(fn, x, recipe, fmt, orient, amax_len):
    rows, cols = x.shape
    x_dtype = fm.IN_BF16 if x.dtype == torch.bfloat16 else fm.IN_FP32
    ldr, ldc = (cols + 15) // 16 * 16, (rows + 15) // 16 * 16
    q_row = torch.full((rows, ldr), 0xAB, dtype=torch.uint8, device="cuda")
    q_col = torch.full((cols, ldc), 0xCD, dtype=torch.uint8, device="cuda")
    shp_r, dt = fm.scale_grid_shape(recipe, rows, cols, fm.ROW)
    shp_c, _ = fm.scale_grid_shape(recipe, rows, cols, fm.COL)
    s_row = torch.zeros(shp_r, dtype=dt, device="cuda") if shp_r else None
    s_col = torch.zeros(shp_c, dtype=dt, device="cuda") if shp_c else None
    scale = torch.ones(1, dtype=torch.float32, device="cuda")
    scale_inv = torch.zeros(1, dtype=torch.float32, device="cuda")
    amax = torch.zeros(amax_len, dtype=torch.float32, device="cuda")
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = fn(x, x_dtype, rows, cols, x.stride(0), recipe, fmt, orient, 0, q_row, ldr, s_row, q_col, ldc, s_col,
            scale, scale_inv, amax, nf)
    assert st == fm.OK, fm.status_string(st)
    torch.cuda.synchronize()
    return q_row, s_row, q_col, s_col, scale, scale_inv, amax[:1], nf


def _same(a, b):
    for u, v in zip(a, b):
        if u is None:
            assert v is None
            continue
        if u.dtype == torch.float32:
            assert same_f32(host(u), host(v))
        else:
            assert torch.equal(u, v)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fmt", [fm.E4M3, fm.E5M2])
def test_static_scratch_matches_fp8_quantize_twice(dtype, fmt):
    """Current scaling: a large tensor (the amax pass uses every partial
    slot), then a smaller one with a 16x smaller amax."""
    need_gpu()
    big = _tensor(4096, 8192, 31, 1.0, dtype)
    small = _tensor(300, 520, 32, 1.0 / 16, dtype)
    for x in (big, small):
        want = _run(fm.fp8_quantize, x, fm.TENSOR_CURRENT, fmt, fm.ROW_AND_COL, fm.AMAX_SLOTS)
        got = _run(fm.fp8_quantize_static_scratch, x, fm.TENSOR_CURRENT, fmt, fm.ROW_AND_COL, 1)
        _same(want, got)
    # the small tensor's amax is its own, not the big one's
    assert host(got[6])[0] == np.float32(small.float().abs().max().item())


def test_static_scratch_strided_input_and_other_recipes():
    """A strided input (the 2-D amax pass) and the recipes that use no
    scratch: the same results as fp8_quantize."""
    need_gpu()
    base = _tensor(1000, 4200, 41, 1.0, torch.bfloat16)
    x = base[:, :4000]
    want = _run(fm.fp8_quantize, x, fm.TENSOR_CURRENT, fm.E4M3, fm.ROW, fm.AMAX_SLOTS)
    got = _run(fm.fp8_quantize_static_scratch, x, fm.TENSOR_CURRENT, fm.E4M3, fm.ROW, 1)
    _same(want, got)
    y = _tensor(384, 640, 42, 1.0, torch.float32)
    for recipe in (fm.BLOCK_1x128, fm.BLOCK_128x128, fm.MX_1x32, fm.CHANNEL):
        want = _run(fm.fp8_quantize, y, recipe, fm.E4M3, fm.ROW_AND_COL, fm.AMAX_SLOTS)
        got = _run(fm.fp8_quantize_static_scratch, y, recipe, fm.E4M3, fm.ROW_AND_COL, fm.AMAX_SLOTS)
        _same(want[:4], got[:4])
