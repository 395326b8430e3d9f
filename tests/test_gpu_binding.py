"""The torch binding checks every tensor against the sizes and dtypes the
kernels will touch before it calls the library (the C entry points take
plain pointers and cannot): a wrong argument is an Fp8Error, raised before
any launch, never an access outside a buffer."""
import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _codes(r, c):
    return torch.zeros(r, c, dtype=torch.uint8, device="cuda")


def test_quantize_argument_checks():
    need_gpu()
    x = torch.zeros(64, 256, dtype=torch.bfloat16, device="cuda")
    for recipe in (fm.TENSOR_CURRENT, fm.TENSOR_DELAYED):
        with pytest.raises(fm.Fp8Error, match="amax"):
            fm.quantize(x, recipe, fm.E4M3, fm.ROW, scale=torch.ones(1, device="cuda"),
                        amax=torch.zeros(1, device="cuda"))
    with pytest.raises(fm.Fp8Error, match="dtype"):
        fm.quantize(x.half(), fm.BLOCK_1x128, fm.E4M3, fm.ROW)
    with pytest.raises(fm.Fp8Error, match="column stride"):
        fm.quantize(x.t(), fm.BLOCK_1x128, fm.E4M3, fm.ROW)
    with pytest.raises(fm.Fp8Error, match="scale"):
        fm.quantize(x, fm.TENSOR_DELAYED, fm.E4M3, fm.ROW, scale=torch.ones(1, dtype=torch.float64, device="cuda"))


@pytest.mark.parametrize("recipe", [fm.GEMM_TENSOR, fm.GEMM_BLOCK_1x128_128x128, fm.GEMM_BLOCK_1x128_1x128,
                                    fm.GEMM_MX_1x32, fm.GEMM_BLOCK_128x128_128x128, fm.GEMM_CHANNEL])
def test_gemm_argument_checks(recipe):
    need_gpu()
    M, N, K = 256, 384, 512
    a, b = _codes(M, K), _codes(N, K)
    n_a, dt = fm._scale_need(recipe, M, K, True)
    n_b, _ = fm._scale_need(recipe, N, K, False)
    s_a = torch.ones(n_a, dtype=dt, device="cuda")
    s_b = torch.ones(n_b, dtype=dt, device="cuda")
    c = fm.gemm(a, fm.E4M3, s_a, b, fm.E4M3, s_b, recipe, K)  # the sizes that fit run
    torch.cuda.synchronize()
    assert c.shape == (M, N)
    bad = [
        dict(c=torch.empty(M, N, dtype=torch.float16, device="cuda")),  # 2-byte output taken for FP32
        dict(c=torch.empty(M, N - 16, dtype=torch.bfloat16, device="cuda")),
        dict(M=M + 1),
        dict(N=N + 16),
        dict(K=K + 16),
        dict(s_a=s_a[: n_a - 1]),
        dict(s_b=s_b[: n_b - 1]),
        dict(s_a=torch.ones(n_a, dtype=torch.float64 if dt == torch.float32 else torch.int8, device="cuda")),
        dict(out_dtype=torch.float16),
    ]
    for kw in bad:
        args = dict(a=a, fmt_a=fm.E4M3, s_a=s_a, b=b, fmt_b=fm.E4M3, s_b=s_b, recipe=recipe, K=K)
        args.update(kw)
        with pytest.raises(fm.Fp8Error):
            fm.gemm(**args)


def test_bf16_gemm_argument_checks():
    need_gpu()
    a = torch.zeros(128, 256, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(64, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fm.Fp8Error, match="dtype"):
        fm.bf16_gemm(a, b, c=torch.empty(128, 64, dtype=torch.float16, device="cuda"))
    with pytest.raises(fm.Fp8Error):
        fm.bf16_gemm(a, b[:, :128])
    with pytest.raises(fm.Fp8Error):
        fm.bf16_gemm(a, b, c=torch.empty(127, 64, dtype=torch.bfloat16, device="cuda"))
