"""The measurement kernels behind the bench line's ceilings
(libfp8mi_probe.so, include/fp8mi_probe.h).  They are not part of the
method, but the bench judges the path's kernels against what they measure,
so they are checked here: each stream moves exactly the bytes its mix names
(also for item counts that leave a ragged last trip), and the MFMA loops
(fixed and varied operands) and the empty kernel run and leave sane
counters."""
import numpy as np
import pytest
import torch

from fp8_scaled_quantization_scale_amd import probe

pytestmark = pytest.mark.gpu

HINTS = [0, probe.NT_LOAD | probe.NT_STORE, probe.BLOCKED, probe.NT_LOAD | probe.NT_STORE | probe.BLOCKED]


def _need():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    probe.load()  # raises if the library is missing


@pytest.mark.parametrize("n16", [2, 4098, 3 * 65536 + 1030])
@pytest.mark.parametrize("hints", HINTS)
def test_stream_mixes_move_the_named_chunks(hints, n16):
    _need()
    g = torch.Generator(device="cuda")
    g.manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda", generator=g)
    chunks = src.view(-1, 4)  # 16-byte chunks
    d0 = torch.zeros_like(src)
    probe.stream(src, d0, None, probe.COPY | hints)
    half = torch.zeros(n16 // 2 * 4, dtype=torch.int32, device="cuda")
    probe.stream(src, half, None, probe.HALF | hints)
    lo, hi = torch.zeros_like(half), torch.zeros_like(half)
    probe.stream(src, lo, hi, probe.SPLIT | hints)
    sentinel = torch.zeros(4, dtype=torch.int32, device="cuda")
    probe.stream(src, sentinel, None, probe.READ | hints)
    torch.cuda.synchronize()
    assert torch.equal(d0, src)
    assert torch.equal(half.view(-1, 4), chunks[0::2] ^ chunks[1::2])
    assert torch.equal(lo.view(-1, 4), chunks[0::2])
    assert torch.equal(hi.view(-1, 4), chunks[1::2])
    assert not sentinel.any()  # READ writes only when the XOR of the data is its sentinel


@pytest.mark.parametrize("varied", [False, True])
def test_mfma_loop_counters(varied):
    _need()
    wgs, iters = 8, 2000
    clocks = torch.zeros(4 * wgs, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    probe.mfma(iters, wgs, clocks, sink, varied)
    torch.cuda.synchronize()
    c = clocks.view(-1, 4).cpu().numpy().astype(np.float64)
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] > c[:, 2]).all()
    ghz = (c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * probe.wall_clock_khz() / 1e6
    assert ((ghz > 0.3) & (ghz < 3.0)).all(), ghz
    # at least the MFMA issue time: iters x 8 products x 32 cycles per wave,
    # two waves sharing each SIMD
    assert ((c[:, 1] - c[:, 0]) >= iters * 8 * 32 * 2 * 0.9).all()
    assert sink.item() == 0.0


def test_empty_launch():
    _need()
    probe.empty(1, 256)
    probe.empty(1024, 64)
    torch.cuda.synchronize()
