"""Pins of the oracle's FP8 formats and encoder to facts outside the oracle:
constants printed on the pages, torch's own float8 dtypes (named on the
"2025 technical guide", sec. 1.1), and exact arithmetic."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_constants.txt")
TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            k, v, tol = line.split()
            out[k] = (float(v), float(tol))
    return out


def _close(value, key, g):
    v, tol = g[key]
    assert abs(value - v) <= tol * abs(v), (key, value, v)


def test_printed_constants():
    g = _golden()
    t5 = oracle.decode_table("e5m2")
    t4 = oracle.decode_table("e4m3")
    _close(oracle.max_value("e5m2"), "e5m2_max", g)
    assert oracle.max_value("e5m2") > g["e5m2_max_lower"][0]
    # smallest normal E5M2: exponent field 1, mantissa 0
    _close(t5[0b00000100], "e5m2_min_normal", g)
    # bias 15: exponent field 15 with mantissa 0 is exactly 1.0
    assert t5[int(g["e5m2_bias"][0]) << 2] == 1.0
    # four steps per binade: 1.0, 1.25, 1.5, 1.75
    steps = int(g["e5m2_steps_per_binade"][0])
    assert list(t5[0x3C:0x3C + steps]) == [1.0, 1.25, 1.5, 1.75]
    assert t5[0x3C + steps] == 2.0
    _close(oracle.max_value("e4m3"), "e4m3_max", g)
    # bit widths: E4M3 has 8 codes per binade, E5M2 4 (3 resp. 2 mantissa bits)
    assert list(t4[0x38:0x40]) == [1 + m / 8 for m in range(8)]
    assert 2 ** int(g["e4m3_mantissa_bits"][0]) == 8
    assert 2 ** int(g["e5m2_mantissa_bits"][0]) == 4
    # exponent fields: E4M3 normal binades 2^-6..2^8 (15 fields), E5M2 2^-14..2^15
    assert t4[0x08] == 2.0 ** -6 and t4[0x78] == 2.0 ** 8
    assert t5[0x04] == 2.0 ** -14 and t5[0x78] == 2.0 ** 15
    # E8M0: 8 exponent bits, no mantissa -> 2^(byte-127), byte 255 is NaN
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_decode_matches_torch_dtype(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
    ours = oracle.decode_table(fmt)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], ours[fin])
    # -0 is code 0x80
    assert np.signbit(ours[0x80]) and ours[0x80] == 0.0


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_roundtrip_all_codes(fmt):
    tab = oracle.decode_table(fmt)
    codes = np.arange(256)
    fin = np.isfinite(tab)
    back = oracle.encode(fmt, tab.astype(np.float32))
    assert np.array_equal(back[fin], codes[fin])
    # NaN codes encode back to the canonical NaN 0x7F; E5M2 +-Inf saturate
    assert np.all(back[np.isnan(tab)] == 0x7F)
    if fmt == "e5m2":
        assert back[0x7C] == 0x7B and back[0xFC] == 0xFB


def _torch_codes(fmt, v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v32).to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_encode_vs_torch_strided_fp32(fmt):
    """A strided sweep of every float32 bit pattern (stride 257, ~16.7M values)
    against torch's round-to-nearest-even cast, wherever |v| <= max.  Beyond
    that, the oracle saturates (checked separately)."""
    mx = oracle.max_value(fmt)
    bits = np.arange(0, 2 ** 32, 257, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    inr = np.abs(v) <= mx  # excludes NaN and out-of-range
    v = np.ascontiguousarray(v[inr])
    assert np.array_equal(oracle.encode(fmt, v), _torch_codes(fmt, v))


def _sweep_chunk(fmt: str, start: int, n: int) -> int:
    """Mismatches of the oracle's encoder over the float32 bit patterns
    [start, start + n): against torch's nearest-even cast where |v| <= max,
    against saturation to +-max beyond (+-Inf included), and against the
    canonical NaN code 0x7F for every NaN pattern."""
    v = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    got = oracle.encode(fmt, v)
    a = np.abs(v)
    inr = a <= oracle.max_value(fmt)
    bad = int(np.count_nonzero(got[inr] != _torch_codes(fmt, np.ascontiguousarray(v[inr]))))
    top = 0x7E if fmt == "e4m3" else 0x7B
    over = a > oracle.max_value(fmt)  # NaN compares false: not in `over`
    want = np.where(np.signbit(v[over]), 0x80 | top, top).astype(np.uint8)
    bad += int(np.count_nonzero(got[over] != want))
    nan = np.isnan(v)
    bad += int(np.count_nonzero(got[nan] != 0x7F))
    assert int(inr.sum() + over.sum() + nan.sum()) == n
    return bad


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_encode_every_fp32_pattern(fmt):
    """All 2^32 float32 inputs: the oracle's nearest-value search equals
    torch's round-to-nearest-even cast (a library routine with its own
    implementation) everywhere inside the format's range, and the closed-form
    saturation / NaN rule outside it.  Chunks run on worker threads (the
    oracle's C loop drops the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    oracle.encode(fmt, np.zeros(1, np.float32))  # fill the oracle's table once
    chunk = 1 << 24
    nthreads = min(8, os.cpu_count() or 1)
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(nthreads) as ex:
            bad = sum(ex.map(lambda c: _sweep_chunk(fmt, c * chunk, chunk), range((1 << 32) // chunk)))
    finally:
        torch.set_num_threads(torch_threads)
    assert bad == 0


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_encode_vs_torch_all_bf16(fmt):
    mx = oracle.max_value(fmt)
    bits = (np.arange(2 ** 16, dtype=np.uint32) << 16)
    v = bits.view(np.float32)
    inr = np.abs(v) <= mx
    v = np.ascontiguousarray(v[inr])
    assert np.array_equal(oracle.encode(fmt, v), _torch_codes(fmt, v))


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_encode_midpoints_and_neighbours(fmt):
    """Every midpoint between adjacent grid values (exact in float32), one ulp
    either side, with both signs: torch agrees, and exact ties go to the even
    code."""
    tab = oracle.decode_table(fmt)
    top = 0x7E if fmt == "e4m3" else 0x7B
    g = tab[: top + 1]
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (g[:-1] + g[1:]) / 2)
    lo = np.nextafter(mids, np.float32(0))
    hi = np.nextafter(mids, np.float32(np.inf))
    vals = np.concatenate([mids, lo, hi]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(oracle.encode(fmt, vals), _torch_codes(fmt, vals))
    # ties to even
    c = oracle.encode(fmt, mids)
    assert np.all(c % 2 == 0)
    assert np.all((c == np.arange(top)) | (c == np.arange(1, top + 1)))
    # just below a midpoint rounds down, just above rounds up
    assert np.array_equal(oracle.encode(fmt, lo[1:]), np.arange(1, top))
    assert np.array_equal(oracle.encode(fmt, hi), np.arange(1, top + 1))


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_encode_saturation_nan_and_signed_zero(fmt):
    mx = np.float32(oracle.max_value(fmt))
    top = 0x7E if fmt == "e4m3" else 0x7B
    big = np.array([mx, np.nextafter(mx, np.float32(np.inf)), mx * 1.5, 3.0e38, np.inf],
                   np.float32)
    assert np.all(oracle.encode(fmt, big) == top)
    assert np.all(oracle.encode(fmt, -big) == (0x80 | top))
    assert np.all(oracle.encode(fmt, np.array([np.nan, -np.nan], np.float32)) == 0x7F)
    assert oracle.encode(fmt, np.array([-0.0], np.float32))[0] == 0x80
    # negative values that round to zero keep the sign
    tiny = np.float32(oracle.decode_table(fmt)[1] / 4)
    assert oracle.encode(fmt, np.array([-tiny, tiny], np.float32)).tolist() == [0x80, 0x00]


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_encode_is_nearest_by_brute_force(fmt):
    """Random in-range values: the chosen code's value is at least as close as
    every other finite code (exhaustive comparison against all 256 codes)."""
    rng = np.random.default_rng(7)
    mx = oracle.max_value(fmt)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 7, 20000))).astype(np.float32)
    v = v[np.abs(v) <= mx]
    c = oracle.encode(fmt, v)
    tab = oracle.decode_table(fmt)
    fin = np.isfinite(tab)
    dist = np.abs(tab[fin][None, :] - v.astype(np.float64)[:, None])
    best = dist.min(axis=1)
    assert np.array_equal(np.abs(tab[c] - v.astype(np.float64)), best)
