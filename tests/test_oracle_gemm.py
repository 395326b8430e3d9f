"""Pins of the oracle's GEMM reference and tolerance check.

The reference is C[i,j] = sum_k a[i,k] b[j,k] over dequantized operands
("2025 technical guide", sec. 3.1: the GEMM inputs are quantized, the
outputs stay BF16/FP32).  It is pinned to exact rational arithmetic on
tiny shapes (which also fixes which index is contracted and which operand
is transposed), to exact special cases, and to its block-scale layout."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _exact_gemm(a, b):
    M, K = a.shape
    N = b.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(a[i, k])) * Fraction(float(b[j, k]))
            out[i][j] = acc
    return out


def test_gemm_ref_against_exact_rationals():
    rng = np.random.default_rng(1)
    M, N, K = 3, 5, 7  # all different: a transposed operand cannot pass
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[qa & 0x7F == 0x7F] = 0x11  # no NaN codes
    qb[qb & 0x7F == 0x7F] = 0x22
    a = oracle.dequant("e4m3", qa, np.float32(0.37))
    b = oracle.dequant("e4m3", qb, np.float32(1.9e-3))
    c, s = oracle.gemm_ref(a, b)
    ex = _exact_gemm(a, b)
    for i in range(M):
        for j in range(N):
            e = ex[i][j]
            assert abs(Fraction(c[i, j]) - e) <= Fraction(s[i, j]) * Fraction(1, 2 ** 50)
    ii, jj = np.array([0, 2, 1]), np.array([4, 0, 3])
    ce, se = oracle.gemm_ref_entries(a, b, ii, jj)
    for t in range(3):
        assert abs(Fraction(ce[t]) - ex[ii[t]][jj[t]]) <= Fraction(se[t]) * Fraction(1, 2 ** 50)


def test_gemm_ref_exact_small_integers():
    """Codes of small integers and power-of-two scales: every partial sum is an
    integer below 2^24, so the float64 result is exact."""
    rng = np.random.default_rng(2)
    M, N, K = 16, 24, 256
    ints = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8], np.float32)
    va = rng.choice(ints, (M, K)) * rng.choice([-1, 1], (M, K))
    vb = rng.choice(ints, (N, K)) * rng.choice([-1, 1], (N, K))
    qa = oracle.encode("e4m3", va.astype(np.float32))
    qb = oracle.encode("e5m2", vb.astype(np.float32))
    a = oracle.dequant("e4m3", qa, np.float32(0.25))
    b = oracle.dequant("e5m2", qb, np.float32(2.0))
    c, _ = oracle.gemm_ref(a, b)
    assert np.array_equal(c, (va.astype(np.int64) @ vb.astype(np.int64).T) * 0.5)


def test_block_grid_expansion():
    """1x128 grid on A (per row, per K block) and 128x128 grid on B."""
    M, N, K = 3, 256, 384
    qa = np.full((M, K), 0x38, np.uint8)  # E4M3 1.0
    qb = np.full((N, K), 0x38, np.uint8)
    ga = np.arange(M * 3, dtype=np.float32).reshape(M, 3) + 1
    gb = np.arange(2 * 3, dtype=np.float32).reshape(2, 3) + 10
    a = oracle.dequant("e4m3", qa, ga, 1, 128)
    b = oracle.dequant("e4m3", qb, gb, 128, 128)
    for i in range(M):
        for k in range(K):
            assert a[i, k] == ga[i, k // 128]
    for j in range(N):
        for k in range(0, K, 61):
            assert b[j, k] == gb[j // 128, k // 128]
    c, _ = oracle.gemm_ref(a, b)
    for i in range(M):
        for j in range(N):
            assert c[i, j] == 128 * sum(ga[i, kb] * gb[j // 128, kb] for kb in range(3))


def test_mx_dequant_uses_power_of_two_scales():
    q = np.full((2, 64), 0x38, np.uint8)
    sb = np.array([[127, 130], [100, 255]], np.uint8)
    d = oracle.dequant_mx("e4m3", q, sb, 1, 32)
    assert np.all(d[0, :32] == 1.0) and np.all(d[0, 32:] == 8.0)
    assert np.all(d[1, :32] == 2.0 ** -27) and np.all(np.isnan(d[1, 32:]))


def test_identity_b_reproduces_a():
    rng = np.random.default_rng(4)
    K = 128
    qa = oracle.encode("e4m3", rng.standard_normal((8, K)).astype(np.float32) * 10)
    qb = np.zeros((K, K), np.uint8)
    np.fill_diagonal(qb, 0x38)
    a = oracle.dequant("e4m3", qa, np.float32(0.5))
    c, _ = oracle.gemm_ref(a, oracle.dequant("e4m3", qb, np.float32(1.0)))
    assert np.array_equal(c, a)


def test_tolerance_check():
    c_ref = np.array([1.0, -2.0, 0.0, np.nan, np.inf])
    s = np.array([1024.0, 1024.0, 1024.0, 1.0, 1.0])
    ok = np.array([1.0 + 0.999, -2.0 - 0.999, 0.5, np.nan, np.inf])
    assert not oracle.gemm_violations(ok, c_ref, s, "fp32").any()
    bad = np.array([1.0 + 1.001, -2.0, 0.0, 1.0, -np.inf])
    assert oracle.gemm_violations(bad, c_ref, s, "fp32").tolist() == [True, False, False, True, True]
    # BF16 output adds 2^-8 |C_ref|
    cr = np.array([256.0])
    assert not oracle.gemm_violations(np.array([257.0]), cr, np.array([0.0]), "bf16").any()
    assert oracle.gemm_violations(np.array([257.5]), cr, np.array([0.0]), "bf16").all()
