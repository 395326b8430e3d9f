"""The C-ABI library loads and exports every entry point include/fp8mi.h
declares; host-side argument validation returns the documented status codes
before any GPU work (runs without a GPU: only invalid calls are made)."""
import os
import re
import subprocess

import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mi.h")

BAD = 0x1000  # never dereferenced: validation fails before any launch
GOOD = 0x10000  # 16-byte aligned stand-in pointer


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fp8_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted(fm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fm.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (fp8_\w+)$", out, flags=re.M))
    assert set(_declared()) <= exported
    assert fm.version() == 500
    assert fm.status_string(fm.ERR_ALIGN).startswith("pointer")


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"^#define FP8MI_(\w+) \(?(-?\d+)\)?", text, flags=re.M))
    assert len(defs) >= 25
    for name, val in defs.items():
        assert getattr(fm, name) == int(val), name
    launch = open(os.path.join(ROOT, "fp8_scaled_quantization_scale_amd", "csrc", "launch.hpp")).read()
    assert int(re.search(r"kAmaxSlots = (\d+);", launch).group(1)) == int(defs["AMAX_SLOTS"])


def _q(**kw):
    args = dict(x=GOOD, x_dtype=fm.IN_BF16, rows=256, cols=256, ld_x=256, recipe=fm.BLOCK_1x128,
                fmt=fm.E4M3, orient=fm.ROW, margin=0, q_row=GOOD, ld_q_row=256, s_row=GOOD,
                q_col=None, ld_q_col=0, s_col=None, scale=None, scale_inv=None, amax=None,
                nonfinite=None, stream=0)
    args.update(kw)
    return fm.fp8_quantize(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(x_dtype=7), fm.ERR_ENUM),
    (dict(recipe=9), fm.ERR_ENUM),
    (dict(fmt=2), fm.ERR_ENUM),
    (dict(orient=0), fm.ERR_ENUM),
    (dict(rows=-1), fm.ERR_SHAPE),
    (dict(margin=65), fm.ERR_SHAPE),
    (dict(x=None), fm.ERR_NULL),
    (dict(q_row=None), fm.ERR_NULL),
    (dict(s_row=None), fm.ERR_NULL),
    (dict(orient=fm.COL), fm.ERR_NULL),
    (dict(ld_x=100), fm.ERR_SHAPE),
    (dict(ld_q_row=128), fm.ERR_SHAPE),
    (dict(x=GOOD + 8), fm.ERR_ALIGN),
    (dict(ld_x=260), fm.ERR_ALIGN),
    (dict(q_row=GOOD + 4), fm.ERR_ALIGN),
    (dict(ld_q_row=264), fm.ERR_ALIGN),
    (dict(recipe=fm.TENSOR_CURRENT), fm.ERR_NULL),
    (dict(recipe=fm.TENSOR_CURRENT, amax=GOOD, scale=GOOD), fm.ERR_NULL),
    (dict(recipe=fm.TENSOR_DELAYED, amax=GOOD), fm.ERR_NULL),
    (dict(recipe=fm.CHANNEL, rows=(1 << 31) * 128, cols=256, ld_x=256), fm.ERR_UNSUPPORTED),
])
def test_quantize_validation(kw, code):
    assert _q(**kw) == code


def test_quantize_empty_is_ok_without_launch():
    assert _q(rows=0) == fm.OK
    assert _q(cols=0, x=None, q_row=None) == fm.OK


def _g(**kw):
    args = dict(a=GOOD, fmt_a=fm.E4M3, s_a=GOOD, lda=256, b=GOOD, fmt_b=fm.E4M3, s_b=GOOD, ldb=256,
                recipe=fm.GEMM_TENSOR, layout=fm.LAYOUT_TN, M=128, N=128, K=256, c=GOOD,
                c_dtype=fm.OUT_BF16, ldc=128, stream=0)
    args.update(kw)
    return fm.fp8_gemm_scaled(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(fmt_a=3), fm.ERR_ENUM),
    (dict(fmt_b=-1), fm.ERR_ENUM),
    (dict(recipe=6), fm.ERR_ENUM),
    (dict(c_dtype=2), fm.ERR_ENUM),
    (dict(M=-1), fm.ERR_SHAPE),
    (dict(c=None), fm.ERR_NULL),
    (dict(a=None), fm.ERR_NULL),
    (dict(s_b=None), fm.ERR_NULL),
    (dict(K=200), fm.ERR_SHAPE),
    (dict(lda=128), fm.ERR_SHAPE),
    (dict(ldc=100), fm.ERR_SHAPE),
    (dict(a=GOOD + 1), fm.ERR_ALIGN),
    (dict(ldb=264 - 4), fm.ERR_ALIGN),
    (dict(s_a=GOOD + 2), fm.ERR_ALIGN),  # scale grids are read in aligned dwords
    (dict(s_b=GOOD + 1, recipe=3), fm.ERR_ALIGN),
    (dict(lda=(1 << 22) + 16), fm.ERR_UNSUPPORTED),
    (dict(M=0x7FFFFFFF, N=0x7FFFFFFF, ldc=0x7FFFFFFF), fm.ERR_UNSUPPORTED),  # tile count past 2^31
    (dict(layout=1), fm.ERR_UNSUPPORTED),  # only the K-contiguous (TN) layout is built
    (dict(layout=-1), fm.ERR_UNSUPPORTED),
    (dict(layout=1, a=None, fmt_a=9), fm.ERR_UNSUPPORTED),  # checked first, before anything else
])
def test_gemm_validation(kw, code):
    assert _g(**kw) == code


def test_gemm_empty_is_ok_without_launch():
    assert _g(M=0) == fm.OK
    assert _g(N=0, c=None) == fm.OK


def test_history_validation():
    f = fm.fp8_amax_history_update
    assert f(GOOD, GOOD, 200, GOOD, 5, 0, GOOD, GOOD, None, 0) == fm.ERR_ENUM
    assert f(None, GOOD, 200, GOOD, 0, 0, GOOD, GOOD, None, 0) == fm.ERR_NULL
    assert f(GOOD, GOOD, 0, GOOD, 0, 0, GOOD, GOOD, None, 0) == fm.ERR_SHAPE
    assert f(GOOD, GOOD, 200, GOOD, 0, -1, GOOD, GOOD, None, 0) == fm.ERR_SHAPE


def _b(**kw):
    args = dict(a=GOOD, lda=256, b=GOOD, ldb=256, M=128, N=128, K=256, c=GOOD, c_dtype=fm.OUT_BF16,
                ldc=128, stream=0)
    args.update(kw)
    return fm.fp8_bf16_gemm(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(c_dtype=2), fm.ERR_ENUM),
    (dict(K=-8), fm.ERR_SHAPE),
    (dict(c=None), fm.ERR_NULL),
    (dict(b=None), fm.ERR_NULL),
    (dict(K=252), fm.ERR_SHAPE),
    (dict(ldb=128), fm.ERR_SHAPE),
    (dict(ldc=64), fm.ERR_SHAPE),
    (dict(a=GOOD + 8), fm.ERR_ALIGN),
    (dict(lda=260), fm.ERR_ALIGN),
    (dict(lda=(1 << 21) + 8), fm.ERR_UNSUPPORTED),
    (dict(M=0x7FFFFFFF, N=0x7FFFFFFF, ldc=0x7FFFFFFF), fm.ERR_UNSUPPORTED),
])
def test_bf16_gemm_validation(kw, code):
    assert _b(**kw) == code


def test_bf16_gemm_empty_is_ok_without_launch():
    assert _b(M=0) == fm.OK
    assert _b(N=0, c=None) == fm.OK


def test_binding_rejects_host_tensors():
    """The kernels read and write every tensor on the GPU: the binding refuses
    host tensors before any library call (a host pointer handed to a kernel
    would be an out-of-bounds access, not an error)."""
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    q = torch.zeros(4, 16, dtype=torch.uint8)
    s1 = torch.ones(1)
    with pytest.raises(fm.Fp8Error, match="device tensor"):
        fm.quantize(x, fm.BLOCK_1x128, fm.E4M3, fm.ROW)
    with pytest.raises(fm.Fp8Error, match="device tensor"):
        fm.gemm(q, fm.E4M3, s1, q, fm.E4M3, s1, fm.GEMM_TENSOR, 16)
    with pytest.raises(fm.Fp8Error, match="device tensor"):
        fm.bf16_gemm(x, x)
    with pytest.raises(fm.Fp8Error, match="device tensors"):
        fm.fp8_gemm_scaled(q, fm.E4M3, s1, 16, q, fm.E4M3, s1, 16, fm.GEMM_TENSOR, fm.LAYOUT_TN, 4, 4, 16,
                           torch.zeros(4, 4), fm.OUT_FP32, 4, stream=0)


# ---------------------------------------------------------------------------
# the measurement library (libfp8mi_probe.so, include/fp8mi_probe.h)
# ---------------------------------------------------------------------------

PROBE_HEADER = os.path.join(ROOT, "include", "fp8mi_probe.h")


def test_probe_library_exports_every_declared_symbol():
    from fp8_scaled_quantization_scale_amd import probe

    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"^\s*\w+\**\s+\**(fp8probe_\w+)\s*\(", text, flags=re.M)))
    assert declared == sorted(probe.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True, text=True).stdout
    assert set(declared) <= set(re.findall(r" T (fp8probe_\w+)$", out, flags=re.M))
    defs = dict(re.findall(r"^#define FP8PROBE_(\w+) (\d+)", open(PROBE_HEADER).read(), flags=re.M))
    assert {k: int(v) for k, v in defs.items()} == {"READ": probe.READ, "COPY": probe.COPY, "HALF": probe.HALF,
                                                     "SPLIT": probe.SPLIT, "NT_LOAD": probe.NT_LOAD,
                                                     "NT_STORE": probe.NT_STORE, "BLOCKED": probe.BLOCKED}


def test_probe_validation():
    from fp8_scaled_quantization_scale_amd import probe

    lib = probe.load()
    assert lib.fp8probe_stream(GOOD, 64, GOOD, None, 9, None) == -2
    assert lib.fp8probe_stream(GOOD, 64, GOOD, None, probe.COPY | 128, None) == -2  # unknown hint bit
    assert lib.fp8probe_stream(GOOD, 63, GOOD, GOOD, probe.HALF | probe.NT_LOAD, None) == -3  # hints keep the checks
    assert lib.fp8probe_stream(GOOD, 0, GOOD, None, probe.COPY | probe.NT_LOAD | probe.NT_STORE, None) == 0
    assert lib.fp8probe_stream(GOOD, 63, GOOD, GOOD, probe.HALF, None) == -3
    assert lib.fp8probe_stream(GOOD, -1, GOOD, None, probe.COPY, None) == -3
    assert lib.fp8probe_stream(None, 64, GOOD, None, probe.COPY, None) == -1
    assert lib.fp8probe_stream(GOOD, 64, GOOD, None, probe.SPLIT, None) == -1
    assert lib.fp8probe_stream(GOOD + 8, 64, GOOD, None, probe.COPY, None) == -5
    assert lib.fp8probe_stream(GOOD, 0, GOOD, None, probe.READ, None) == 0
    assert lib.fp8probe_empty(0, 256, None) == -3
    assert lib.fp8probe_empty(1, 0, None) == -3
    assert lib.fp8probe_empty(1, 1025, None) == -3
    assert lib.fp8probe_mfma(0, 4, GOOD, GOOD, None) == -3
    assert lib.fp8probe_mfma(10, 4, None, GOOD, None) == -1
    assert lib.fp8probe_mfma_varied(0, 4, GOOD, GOOD, None) == -3
    assert lib.fp8probe_mfma_varied(10, 0, GOOD, GOOD, None) == -3
    assert lib.fp8probe_mfma_varied(10, 4, GOOD, None, None) == -1
