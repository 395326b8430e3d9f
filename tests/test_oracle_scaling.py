"""Pins of the oracle's scale rules and recipes.

Scale from amax: the correctly-rounded property is checked with exact
rational arithmetic over every BF16 amax; recipes are checked against
torch's float8 casts applied to torch's own float32 arithmetic (the library
special case), block partition invariants, closed forms for powers of two,
and the history-window behaviour the "2025 technical guide", sec. 2.1 fixes
(200 steps, the maximum of the buffer)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

TORCH_DT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FLT_MAX = np.float32(np.finfo(np.float32).max)


def _is_rn(c: np.float32, exact: Fraction) -> bool:
    """c is the float32 nearest to `exact` (ties: even significand)."""
    lo = np.nextafter(c, np.float32(-np.inf))
    hi = np.nextafter(c, np.float32(np.inf))
    d = abs(Fraction(float(c)) - exact)
    if d > abs(Fraction(float(lo)) - exact) or d > abs(Fraction(float(hi)) - exact):
        return False
    if d == abs(Fraction(float(lo)) - exact) or d == abs(Fraction(float(hi)) - exact):
        return int(np.array(c).view(np.uint32)) % 2 == 0
    return True


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_scale_is_correctly_rounded_for_every_bf16_amax(fmt):
    mx = Fraction(oracle.max_value(fmt))
    bits = (np.arange(0, 0x7F80, dtype=np.uint32) << 16)  # +0 .. largest finite
    amaxes = bits.view(np.float32)
    for a in amaxes[::3]:
        s, si, flag = oracle.scale_from_amax(fmt, a)
        assert flag == 0
        if a == 0:
            assert s == 1 and si == 1
            continue
        q = mx / Fraction(float(a))
        if q > Fraction(float(FLT_MAX)) * (1 + Fraction(1, 2 ** 25)):
            assert s == FLT_MAX  # +Inf quotient is clamped
        else:
            assert _is_rn(s, q), (a, s)
        assert _is_rn(si, 1 / Fraction(float(s))), (a, s, si)


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_scale_closed_forms_and_special_cases(fmt):
    mx = oracle.max_value(fmt)
    for k in range(-100, 100):
        s, si, _ = oracle.scale_from_amax(fmt, np.float32(mx * 2.0 ** k))
        assert s == np.float32(2.0 ** -k) and si == np.float32(2.0 ** k)
    # amax == max: s = 1 and the recipe is a plain saturating cast
    assert oracle.scale_from_amax(fmt, mx)[:2] == (1.0, 1.0)
    # margin m divides the scale by 2^m [From FP16 to FP8, sec. 3.3]
    for m in range(4):
        s, si, _ = oracle.scale_from_amax(fmt, np.float32(3.0), margin=m)
        s0, _, _ = oracle.scale_from_amax(fmt, np.float32(3.0))
        assert s == np.float32(s0 / 2 ** m)
    for bad in (np.inf, np.nan):
        s, si, flag = oracle.scale_from_amax(fmt, np.float32(bad))
        assert (s, si, flag) == (1.0, 1.0, 1)
    s, si, _ = oracle.scale_from_amax(fmt, np.float32(2.0 ** -133))
    assert s == FLT_MAX


def _torch_current(fmt, x_bf16):
    """Per-tensor current scaling spelled with torch float32 ops and torch's
    float8 cast (only valid where no product exceeds max by half an ulp)."""
    xf = x_bf16.float()
    amax = xf.abs().max()
    s = torch.tensor(oracle.max_value(fmt), dtype=torch.float32) / amax
    q = (xf * s).to(TORCH_DT[fmt]).view(torch.uint8)
    return q.numpy(), np.float32(s.item()), np.float32((1.0 / s).item()), np.float32(amax.item())


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_current_scaling_matches_torch(fmt):
    t = workloads.Tensor("X", 64, 256, "outliers", 1.0, 99, 0.03, 50.0)
    x = workloads.make(t)
    q, s, si, am, flag = oracle.quantize_current(fmt, x)
    tq, ts, tsi, tam = _torch_current(fmt, x)
    assert flag == 0 and am == tam and s == ts and si == tsi
    assert np.array_equal(q, tq)


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_delayed_cast_matches_torch(fmt):
    x = workloads.make(workloads.Tensor("G", 32, 160, "normal", 1e-4, 5))
    s = np.float32(3.1e6) if fmt == "e4m3" else np.float32(2.9e8)
    q, am = oracle.quantize_delayed(fmt, x, s)
    xf = x.float()
    prod = xf * torch.tensor(s)
    mx = oracle.max_value(fmt)
    sat = prod.abs() >= mx
    tq = prod.clamp(-mx, mx).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    assert am == np.float32(xf.abs().max().item())
    assert np.array_equal(q, tq)
    assert sat.any()  # the carried-over scale saturates some values here


def _torch_blocks(fmt, x_bf16, br, bc):
    xf = x_bf16.float()
    R, C = xf.shape
    mx = oracle.max_value(fmt)
    q = np.empty((R, C), np.uint8)
    grid = np.empty(((R + br - 1) // br, (C + bc - 1) // bc), np.float32)
    for bi in range(grid.shape[0]):
        for bj in range(grid.shape[1]):
            blk = xf[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            a = blk.abs().max()
            s = torch.tensor(1.0) if a == 0 else torch.tensor(mx, dtype=torch.float32) / a
            q[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc] = (
                (blk * s).to(TORCH_DT[fmt]).view(torch.uint8).numpy())
            grid[bi, bj] = (1.0 / s).item()
    return q, grid


@pytest.mark.parametrize("br,bc", [(1, 128), (128, 1), (128, 128)])
def test_block_scaling_matches_torch_with_ragged_edges(br, bc):
    # 200 x 300 leaves partial blocks at the bottom and right edges
    x = workloads.make(workloads.Tensor("X", 200, 300, "outliers", 1.0, 11, 0.02, 50.0))
    x[3, :] = 0  # whole-zero row: 1x128 blocks with amax 0 get s = 1
    q, grid, bad = oracle.quantize_blocks("e4m3", x, br, bc)
    tq, tgrid = _torch_blocks("e4m3", x, br, bc)
    assert bad == 0
    assert np.array_equal(grid, tgrid)
    assert np.array_equal(q, tq)


def test_block_partition_invariants():
    x = workloads.make(workloads.Tensor("X", 256, 384, "gains", 1.0, 12))
    # each 1x128 block equals current scaling of that sub-tensor
    q, grid, _ = oracle.quantize_blocks("e4m3", x, 1, 128)
    for i, j in [(0, 0), (7, 2), (255, 1)]:
        sub = x[i:i + 1, 128 * j:128 * (j + 1)]
        sq, s, si, _, _ = oracle.quantize_current("e4m3", sub)
        assert np.array_equal(q[i:i + 1, 128 * j:128 * (j + 1)], sq) and grid[i, j] == si
    # column orientation is row orientation of the transpose
    qc, gc, _ = oracle.quantize_blocks("e4m3", x, 128, 1)
    qt, gt, _ = oracle.quantize_blocks("e4m3", x.t().contiguous(), 1, 128)
    assert np.array_equal(qc.T, qt) and np.array_equal(gc.T, gt)
    # 128x128 tiles commute with transposition
    q2, g2, _ = oracle.quantize_blocks("e4m3", x, 128, 128)
    q2t, g2t, _ = oracle.quantize_blocks("e4m3", x.t().contiguous(), 128, 128)
    assert np.array_equal(q2.T, q2t) and np.array_equal(g2.T, g2t)
    # a whole-tensor block is per-tensor current scaling
    qa, ga, _ = oracle.quantize_blocks("e4m3", x, 256, 384)
    qb, _, sib, _, _ = oracle.quantize_current("e4m3", x)
    assert np.array_equal(qa, qb) and ga[0, 0] == sib


def test_nonfinite_inputs():
    x = workloads.make(workloads.Tensor("X", 4, 256, "normal", 1.0, 13))
    x[1, 5] = float("nan")
    x[2, 200] = float("inf")
    q, s, si, am, flag = oracle.quantize_current("e4m3", x)
    assert np.isnan(am) and flag == 1 and s == 1.0 and si == 1.0
    assert q[1, 5] == 0x7F and q[2, 200] == 0x7E
    q, grid, bad = oracle.quantize_blocks("e4m3", x, 1, 128)
    assert bad == 2 and grid[1, 0] == 1.0 and grid[2, 1] == 1.0
    # untouched blocks are unaffected
    q0, g0, _ = oracle.quantize_blocks("e4m3", x[:1], 1, 128)
    assert np.array_equal(q[:1], q0) and np.array_equal(grid[:1], g0)


# ---------------------------------------------------------------------------
# MX [2025 technical guide sec. 2.3; Mastering FP8 LLM training, strategy 4]
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_mx_scale_is_smallest_non_saturating_power_of_two(fmt):
    mx = Fraction(oracle.max_value(fmt))
    bits = (np.arange(1, 0x7F80, 5, dtype=np.uint32) << 16)
    for a in bits.view(np.float32):
        b = oracle.mx_scale_byte(fmt, a)
        e = b - 127
        fa = Fraction(float(a))
        if -127 < e < 127:
            assert fa * Fraction(2) ** -e <= mx < fa * Fraction(2) ** -(e - 1), (a, b)
        elif e == -127:  # clamped: even 2^-127 would leave headroom
            assert fa * Fraction(2) ** 127 <= mx
    for k in range(-100, 100):
        assert oracle.mx_scale_byte(fmt, np.float32(float(mx) * 2.0 ** k)) == 127 + k
    assert oracle.mx_scale_byte(fmt, 0.0) == 127
    assert oracle.mx_scale_byte(fmt, np.inf) == 255
    assert oracle.mx_scale_byte(fmt, np.nan) == 255


@pytest.mark.parametrize("br,bc", [(1, 32), (32, 1)])
def test_mx_quantize_matches_torch(br, bc):
    x = workloads.make(workloads.Tensor("X", 96, 200, "outliers", 1.0, 14, 0.01, 100.0))
    x[0, :32] = 0
    q, sb, bad = oracle.quantize_mx("e4m3", x, br, bc)
    assert bad == 0
    xf = x.float().numpy()
    for bi in range(sb.shape[0]):
        for bj in range(sb.shape[1]):
            blk = xf[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            e = int(sb[bi, bj]) - 127
            assert np.abs(blk).max() * 2.0 ** -e <= 448.0
            scaled = torch.from_numpy(np.ascontiguousarray(blk)) * torch.tensor(2.0 ** -e)
            tq = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc], tq)
    assert sb[0, 0] == 127 if br == 1 else True


@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_mx_floor_rule_closed_form(fmt):
    """OCP floor rule: e = floor(log2 amax) - emax (emax 8 for E4M3, 15 for
    E5M2), computed here from Python's exact frexp, clamped to [-127, 127]."""
    emax = 8 if fmt == "e4m3" else 15
    bits = (np.arange(1, 0x7F80, 3, dtype=np.uint32) << 16)
    for a in bits.view(np.float32):
        _, E = np.frexp(np.float64(a))  # a = f 2^E, f in [0.5, 1)
        e = min(max(int(E) - 1 - emax, -127), 127)
        assert oracle.mx_scale_byte(fmt, a, "floor") == e + 127, a
        # the two rules differ exactly when the significand exceeds max's
        ceil_b = oracle.mx_scale_byte(fmt, a)
        f = np.float64(a) / 2.0 ** (int(E) - 1)
        if -127 < e < 126:
            assert ceil_b - (e + 127) == (1 if f > 1.75 else 0), a
    assert oracle.mx_scale_byte(fmt, 0.0, "floor") == 127
    assert oracle.mx_scale_byte(fmt, np.nan, "floor") == 255


def test_mx_floor_rule_saturates_the_top_binade():
    """A block whose amax lies in (448, 512) keeps e = 0 under the floor rule:
    those elements saturate to 448 (code 0x7E), the ceil rule halves them."""
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [480.0, -500.0, 448.0, 1.0]
    qf, bf, _ = oracle.quantize_mx("e4m3", x, 1, 32, "floor")
    qc, bc, _ = oracle.quantize_mx("e4m3", x, 1, 32)
    assert bf[0, 0] == 127 and bc[0, 0] == 128
    assert list(qf[0, :4]) == [0x7E, 0xFE, 0x7E, oracle.encode("e4m3", np.float32([1.0]))[0]]
    assert list(oracle.decode("e4m3", qc[0, :4])) == [240.0, -256.0, 224.0, 0.5]


def test_channel_scaling_is_current_scaling_per_row():
    """One scale per row: each row equals per-tensor current scaling of that
    row alone; per-column scales are the rows of the transpose."""
    x = workloads.make(workloads.Tensor("X", 64, 520, "gains", 1.0, 15))
    x[5, :] = 0
    q, si, bad = oracle.quantize_channel("e4m3", x)
    assert bad == 0 and si.shape == (64,) and si[5] == 1.0
    for r in (0, 5, 17, 63):
        qr, _, sir, _, _ = oracle.quantize_current("e4m3", x[r:r + 1])
        assert np.array_equal(q[r:r + 1], qr) and si[r] == sir
    qt, sit, _ = oracle.quantize_channel("e5m2", x.t().contiguous())
    for c in (0, 300, 519):
        qc, _, sic, _, _ = oracle.quantize_current("e5m2", x[:, c:c + 1])
        assert np.array_equal(qt[c], qc[:, 0]) and sit[c] == sic


# ---------------------------------------------------------------------------
# amax history [2025 technical guide sec. 2.1; From FP16 to FP8 sec. 3.3]
# ---------------------------------------------------------------------------

def test_history_constant_amax():
    h = oracle.History("e5m2")
    assert h.scale == 1.0
    h.update(np.float32(3.0e-4))
    s, si, _ = oracle.scale_from_amax("e5m2", np.float32(3.0e-4))
    assert h.scale == s and h.scale_inv == si


def test_history_window_is_200_steps():
    h = oracle.History("e5m2", length=200)
    seq = [np.float32(1.0 - 1e-3 * t) for t in range(450)]  # strictly decreasing
    scales = []
    for a in seq:
        h.update(a)
        scales.append(h.scale)
    # while step 0's amax is in the window it is the max; it leaves at step 200
    s0 = oracle.scale_from_amax("e5m2", seq[0])[0]
    assert all(s == s0 for s in scales[:200])
    assert scales[200] == oracle.scale_from_amax("e5m2", seq[1])[0]
    for t in range(200, 450):
        assert scales[t] == oracle.scale_from_amax("e5m2", seq[t - 199])[0]


def test_history_skips_nonfinite_and_restores():
    rng = np.random.default_rng(3)
    amaxes = rng.uniform(1e-5, 1e-3, 400).astype(np.float32)
    amaxes[17] = np.nan
    amaxes[230] = np.inf
    a = oracle.History("e5m2")
    for v in amaxes:
        a.update(v)
    assert a.nonfinite[0] == 2
    b = oracle.History("e5m2")
    for v in amaxes[:200]:
        b.update(v)
    saved = b.state()
    c = oracle.History("e5m2")
    c.ring[:] = saved[0]
    c.head[0] = saved[1]
    c.nonfinite[0] = saved[4]
    for v in amaxes[200:]:
        c.update(v)
    assert np.array_equal(a.ring, c.ring) and a.head[0] == c.head[0]
    assert a.scale == c.scale and a.scale_inv == c.scale_inv


def test_history_head_outside_the_ring_is_taken_modulo_len():
    # The pages fix a ring of the last N amaxes but not what a stored head
    # outside [0, N) means (state saved with another length); the C ABI's
    # reading, which the oracle follows, is head mod N.  Pinned by hand for
    # N = 5: the amax lands in slot (head mod 5) and the head moves one on.
    for head, slot in ((7, 2), (-1, 4), (12, 2), (5, 0), (-6, 4)):
        h = oracle.History("e4m3", 5)
        h.head[0] = head
        h.update(np.float32(3.0))
        want = np.zeros(5, np.float32)
        want[slot] = 3.0
        assert np.array_equal(h.ring, want), head
        assert h.head[0] == (slot + 1) % 5, head
    # a non-finite amax pushes nothing and leaves the stored head as it was
    h = oracle.History("e4m3", 5)
    h.head[0] = 7
    h.update(np.float32(np.nan))
    assert h.head[0] == 7 and not h.ring.any() and h.nonfinite[0] == 1
