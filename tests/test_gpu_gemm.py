"""GPU parity of fp8_gemm_scaled against the oracle's float64 reference.

Operand codes and scales are made by the oracle from seeded BF16 inputs and
uploaded, so nothing the reference sees comes from the HIP path.  Bound:
|C - C_ref| <= 2^-10 sum_k |a b| (+ 2^-8 |C_ref| for BF16 output).  Exact
cases (small integers, power-of-two scales) are compared bit for bit."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm
import oracle
import workloads
from gpu_util import FMT_NAME, dev, host, need_gpu, padded_codes

pytestmark = pytest.mark.gpu

OUT = {fm.OUT_BF16: ("bf16", torch.bfloat16), fm.OUT_FP32: ("fp32", torch.float32)}


def _operands(recipe, M, N, K, fa, fb, seed):
    """Oracle-quantized A [M x K], B [N x K]: (codes, device scales, dequantized)."""
    xa = workloads.make(workloads.Tensor("A", M, K, "outliers", 1.0, seed, 0.02, 50.0)).float().numpy()
    xb = workloads.make(workloads.Tensor("B", N, K, "normal", 0.02, seed + 1)).float().numpy()
    na, nb = FMT_NAME[fa], FMT_NAME[fb]
    if recipe == fm.GEMM_TENSOR:
        qa, _, sia, _, _ = oracle.quantize_current(na, xa)
        qb, _, sib, _, _ = oracle.quantize_current(nb, xb)
        da, db = oracle.dequant(na, qa, sia), oracle.dequant(nb, qb, sib)
        sa, sb = dev(np.array([sia], np.float32)), dev(np.array([sib], np.float32))
    elif recipe == fm.GEMM_BLOCK_1x128_128x128:
        qa, ga, _ = oracle.quantize_blocks(na, xa, 1, 128)
        qb, gb, _ = oracle.quantize_blocks(nb, xb, 128, 128)
        da, db = oracle.dequant(na, qa, ga, 1, 128), oracle.dequant(nb, qb, gb, 128, 128)
        sa, sb = dev(ga), dev(gb)
    elif recipe == fm.GEMM_BLOCK_128x128_128x128:
        qa, ga, _ = oracle.quantize_blocks(na, xa, 128, 128)
        qb, gb, _ = oracle.quantize_blocks(nb, xb, 128, 128)
        da, db = oracle.dequant(na, qa, ga, 128, 128), oracle.dequant(nb, qb, gb, 128, 128)
        sa, sb = dev(ga), dev(gb)
    elif recipe == fm.GEMM_CHANNEL:
        qa, ga, _ = oracle.quantize_channel(na, xa)
        qb, gb, _ = oracle.quantize_channel(nb, xb)
        da, db = oracle.dequant(na, qa, ga[:, None], 1, K), oracle.dequant(nb, qb, gb[:, None], 1, K)
        sa, sb = dev(ga), dev(gb)
    elif recipe == fm.GEMM_BLOCK_1x128_1x128:
        qa, ga, _ = oracle.quantize_blocks(na, xa, 1, 128)
        qb, gb, _ = oracle.quantize_blocks(nb, xb, 1, 128)
        da, db = oracle.dequant(na, qa, ga, 1, 128), oracle.dequant(nb, qb, gb, 1, 128)
        sa, sb = dev(ga), dev(gb)
    else:
        qa, ga, _ = oracle.quantize_mx(na, xa, 1, 32)
        qb, gb, _ = oracle.quantize_mx(nb, xb, 1, 32)
        da, db = oracle.dequant_mx(na, qa, ga, 1, 32), oracle.dequant_mx(nb, qb, gb, 1, 32)
        sa, sb = dev(ga), dev(gb)
    return padded_codes(qa), sa, da, padded_codes(qb), sb, db


def _check(c, da, db, out):
    c_ref, s = oracle.gemm_ref(da, db)
    got = host(c.float())
    bad = oracle.gemm_violations(got, c_ref, s, out)
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5])


RECIPES = [fm.GEMM_TENSOR, fm.GEMM_BLOCK_1x128_128x128, fm.GEMM_BLOCK_1x128_1x128, fm.GEMM_MX_1x32,
           fm.GEMM_BLOCK_128x128_128x128, fm.GEMM_CHANNEL]
SHAPES = [(128, 256, 512), (200, 300, 400), (256, 512, 1024), (17, 33, 144), (513, 129, 256)]


@pytest.mark.parametrize("recipe", RECIPES)
@pytest.mark.parametrize("fa,fb", [(fm.E4M3, fm.E4M3), (fm.E5M2, fm.E4M3), (fm.E4M3, fm.E5M2), (fm.E5M2, fm.E5M2)])
@pytest.mark.parametrize("out", [fm.OUT_BF16, fm.OUT_FP32])
def test_gemm_matches_reference(recipe, fa, fb, out):
    need_gpu()
    name, dt = OUT[out]
    for i, (M, N, K) in enumerate(SHAPES):
        a, sa, da, b, sb, db = _operands(recipe, M, N, K, fa, fb, 1000 + 10 * i)
        c = fm.gemm(a, fa, sa, b, fb, sb, recipe, K, dt, M=M, N=N)
        _check(c, da, db, name)


# K steps of 128 bytes that fill several four-step scale groups and end in a
# partial one (KT = 10 and 14), MX rows whose E8M0 bytes start mid-dword
# (ceil(K / 32) = 37 and 53 bytes per row), ragged tile edges in M and N, and
# (4352 x 4352: 289 output tiles) more tiles than workgroups, so that
# workgroups carry their scale and stage state from one tile to the next.
WALK_SHAPES = [(4352, 4352, 1168), (300, 700, 1680)]


@pytest.mark.parametrize("recipe", RECIPES)
def test_gemm_scale_groups_and_tile_walk(recipe):
    need_gpu()
    for i, (M, N, K) in enumerate(WALK_SHAPES):
        fa, fb, out = (fm.E4M3, fm.E4M3, fm.OUT_BF16) if i == 0 else (fm.E5M2, fm.E4M3, fm.OUT_FP32)
        name, dt = OUT[out]
        a, sa, da, b, sb, db = _operands(recipe, M, N, K, fa, fb, 2000 + 10 * i)
        c = fm.gemm(a, fa, sa, b, fb, sb, recipe, K, dt, M=M, N=N)
        _check(c, da, db, name)


def test_tiny_blockwise_config_in_full():
    """The tiny blockwise workload: A 128 x 512 (1% outlier columns x50) in
    1x128 tiles, B 512 x 256 N(0, 0.02) in 128 x 128 tiles, BF16 out."""
    need_gpu()
    cfg = workloads.CONFIGS["tiny_block"]
    x = workloads.make(cfg.X).float().numpy()
    w = workloads.make(cfg.W).float().numpy()
    qa, ga, _ = oracle.quantize_blocks("e4m3", x, 1, 128)
    qb, gb, _ = oracle.quantize_blocks("e4m3", w, 128, 128)
    c = fm.gemm(padded_codes(qa), fm.E4M3, dev(ga), padded_codes(qb), fm.E4M3, dev(gb),
                fm.GEMM_BLOCK_1x128_128x128, cfg.K, torch.bfloat16, M=cfg.M, N=cfg.N)
    _check(c, oracle.dequant("e4m3", qa, ga, 1, 128), oracle.dequant("e4m3", qb, gb, 128, 128), "bf16")


@pytest.mark.parametrize("recipe", RECIPES)
def test_exact_small_integer_products(recipe):
    """Codes of small integers, power-of-two scales: every partial sum is an
    exact integer < 2^24, so any correct FP32 accumulation gives C exactly."""
    need_gpu()
    rng = np.random.default_rng(5)
    M, N, K = 160, 272, 384
    ints = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8], np.float32)
    va = (rng.choice(ints, (M, K)) * rng.choice([-1, 1], (M, K))).astype(np.float32)
    vb = (rng.choice(ints, (N, K)) * rng.choice([-1, 1], (N, K))).astype(np.float32)
    qa, qb = oracle.encode("e4m3", va), oracle.encode("e5m2", vb)
    if recipe == fm.GEMM_TENSOR:
        ga, gb = np.array([0.5], np.float32), np.array([4.0], np.float32)
        da, db = oracle.dequant("e4m3", qa, ga[0]), oracle.dequant("e5m2", qb, gb[0])
    elif recipe == fm.GEMM_CHANNEL:
        ga = (2.0 ** rng.integers(-2, 3, M)).astype(np.float32)
        gb = (2.0 ** rng.integers(-2, 3, N)).astype(np.float32)
        da, db = oracle.dequant("e4m3", qa, ga[:, None], 1, K), oracle.dequant("e5m2", qb, gb[:, None], 1, K)
    elif recipe == fm.GEMM_BLOCK_128x128_128x128:
        ga = (2.0 ** rng.integers(-2, 3, ((M + 127) // 128, K // 128))).astype(np.float32)
        gb = (2.0 ** rng.integers(-2, 3, ((N + 127) // 128, K // 128))).astype(np.float32)
        da, db = oracle.dequant("e4m3", qa, ga, 128, 128), oracle.dequant("e5m2", qb, gb, 128, 128)
    elif recipe == fm.GEMM_MX_1x32:
        ga = rng.integers(125, 130, (M, K // 32)).astype(np.uint8)
        gb = rng.integers(125, 130, (N, K // 32)).astype(np.uint8)
        da, db = oracle.dequant_mx("e4m3", qa, ga, 1, 32), oracle.dequant_mx("e5m2", qb, gb, 1, 32)
    else:
        ga = (2.0 ** rng.integers(-2, 3, (M, K // 128))).astype(np.float32)
        if recipe == fm.GEMM_BLOCK_1x128_128x128:
            gb = (2.0 ** rng.integers(-2, 3, ((N + 127) // 128, K // 128))).astype(np.float32)
            db = oracle.dequant("e5m2", qb, gb, 128, 128)
        else:
            gb = (2.0 ** rng.integers(-2, 3, (N, K // 128))).astype(np.float32)
            db = oracle.dequant("e5m2", qb, gb, 1, 128)
        da = oracle.dequant("e4m3", qa, ga, 1, 128)
    c_ref, _ = oracle.gemm_ref(da, db)
    args = (padded_codes(qa), fm.E4M3, dev(ga), padded_codes(qb), fm.E5M2, dev(gb), recipe, K)
    c32 = host(fm.gemm(*args, torch.float32, M=M, N=N))
    assert np.array_equal(c32.astype(np.float64), c_ref)
    c16 = fm.gemm(*args, torch.bfloat16, M=M, N=N)
    want = torch.from_numpy(c_ref.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(c16.cpu(), want)


def test_k_zero_writes_zeros():
    need_gpu()
    c = torch.full((40, 50), 7.0, dtype=torch.float32, device="cuda")
    st = fm.fp8_gemm_scaled(None, fm.E4M3, None, 16, None, fm.E4M3, None, 16, fm.GEMM_TENSOR, fm.LAYOUT_TN,
                            40, 50, 0, c, fm.OUT_FP32, 50)
    assert st == fm.OK
    assert torch.count_nonzero(c).item() == 0


def test_ldc_and_strided_output():
    need_gpu()
    M, N, K = 100, 150, 256
    a, sa, da, b, sb, db = _operands(fm.GEMM_BLOCK_1x128_1x128, M, N, K, fm.E4M3, fm.E4M3, 77)
    big = torch.full((M, 200), -1.0, dtype=torch.float32, device="cuda")
    fm.gemm(a, fm.E4M3, sa, b, fm.E4M3, sb, fm.GEMM_BLOCK_1x128_1x128, K, M=M, N=N, c=big)
    _check(big[:, :N], da, db, "fp32")
    assert torch.all(big[:, N:] == -1.0)


# ---------------------------------------------------------------------------
# the BF16 GEMM the FP8 speedup is measured against
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("out", [fm.OUT_BF16, fm.OUT_FP32])
def test_bf16_gemm_matches_reference(out):
    """BF16 operands are exact in float64, so C_ref is their float64 product."""
    need_gpu()
    name, dt = OUT[out]
    for i, (M, N, K) in enumerate(SHAPES + [(300, 520, 2056)]):
        a = workloads.make(workloads.Tensor("A", M, K, "outliers", 1.0, 2000 + i, 0.02, 50.0))
        b = workloads.make(workloads.Tensor("B", N, K, "normal", 0.02, 2100 + i))
        c = fm.bf16_gemm(a.cuda(), b.cuda(), dt)
        _check(c, a.double().numpy(), b.double().numpy(), name)


def test_bf16_gemm_exact_small_integers_and_padding():
    """Small-integer operands (exact FP32 sums) compared bit for bit, with
    padded leading dimensions whose padding holds large values."""
    need_gpu()
    rng = np.random.default_rng(9)
    M, N, K = 272, 144, 392
    va = rng.integers(-8, 9, (M, K + 24)).astype(np.float32)
    vb = rng.integers(-8, 9, (N, K + 8)).astype(np.float32)
    va[:, K:] = 3e4
    vb[:, K:] = -3e4
    a = torch.from_numpy(va).to(torch.bfloat16).cuda()
    b = torch.from_numpy(vb).to(torch.bfloat16).cuda()
    c = torch.empty(M, N, dtype=torch.float32, device="cuda")
    st = fm.fp8_bf16_gemm(a, K + 24, b, K + 8, M, N, K, c, fm.OUT_FP32, N)
    assert st == fm.OK
    want = va[:, :K].astype(np.float64) @ vb[:, :K].astype(np.float64).T
    assert np.array_equal(host(c).astype(np.float64), want)
