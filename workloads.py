"""Seeded synthetic inputs shared by the tests, the oracle checks and bench.py.

This module only draws random numbers and rounds them to BF16; it holds none
of the quantization or GEMM arithmetic.  Both the HIP path and the oracle are
fed the same BF16 bytes made here.

The shapes are the Llama-3 layer shapes the scaled FP8 GEMMs run at; weights
are stored [out x in] (N x K), so every GEMM operand has its contraction
index contiguous.  The pages train on real data and weights; these draws stand
in for them:
  * "normal":   N(0, sigma), sigma is the standard deviation;
  * "outliers": N(0, sigma) with round(frac * cols) whole columns (channels),
                chosen by a seeded permutation, multiplied by `factor`;
  * "gains":    N(0, sigma) * exp(z_k), one log-normal(0, 1) gain per column.
Values are drawn in float32 and rounded to BF16 (nearest-even) last.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Tensor:
    name: str
    rows: int
    cols: int
    kind: str  # normal | outliers | gains
    sigma: float
    seed: int
    frac: float = 0.0
    factor: float = 1.0


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make(t: Tensor, device: str = "cpu", rows: int | None = None) -> torch.Tensor:
    """BF16 tensor [rows x t.cols] for the recipe `t` (rows defaults to t.rows;
    a different row count is a different draw, not a slice of the full one)."""
    r = t.rows if rows is None else rows
    x = torch.randn(r, t.cols, generator=_gen(t.seed, device), device=device,
                    dtype=torch.float32)
    x.mul_(t.sigma)
    if t.kind == "outliers":
        n_out = int(round(t.frac * t.cols))
        perm = torch.randperm(t.cols, generator=_gen(t.seed + 10, "cpu"))[:n_out]
        x[:, perm.to(device)] *= t.factor
    elif t.kind == "gains":
        z = torch.randn(t.cols, generator=_gen(t.seed + 11, "cpu"), dtype=torch.float32)
        x.mul_(torch.exp(z).to(device))
    elif t.kind != "normal":
        raise ValueError(t.kind)
    return x.to(torch.bfloat16)


def outlier_columns(t: Tensor) -> torch.Tensor:
    n_out = int(round(t.frac * t.cols))
    return torch.randperm(t.cols, generator=_gen(t.seed + 10, "cpu"))[:n_out]


@dataclass(frozen=True)
class Config:
    name: str
    recipe: str  # tensor | block | mx
    M: int
    N: int
    K: int
    X: Tensor
    W: Tensor  # stored [N x K]
    G: Tensor | None  # [M x N]
    history_draws: int = 0
    history_seed0: int = 2100
    gemms: tuple = field(default=("fprop",))


def _cfg(c: int, name, recipe, M, N, K, x, w, g, **kw) -> Config:
    base = 1000 * c
    X = Tensor("X", M, K, x[0], x[1], base + 1, *x[2:])
    W = Tensor("W", N, K, w[0], w[1], base + 2, *w[2:])
    G = None if g is None else Tensor("G", M, N, g[0], g[1], base + 3, *g[2:])
    return Config(name, recipe, M, N, K, X, W, G, **kw)


CONFIGS = {
    # blockwise, tiny: A 128x512 with 1% outlier columns x50, B 512x256 N(0,0.02)
    "tiny_block": _cfg(1, "tiny_block", "block", 128, 256, 512,
                       ("outliers", 1.0, 0.01, 50.0), ("normal", 0.02), None),
    # per-tensor hybrid at the Llama-3-8B attention projection
    "llama3_8b_attn_tensor": _cfg(2, "llama3_8b_attn_tensor", "tensor", 8192, 4096, 4096,
                                  ("gains", 1.0), ("normal", 0.02), ("normal", 1e-4),
                                  history_draws=200, gemms=("fprop", "dgrad")),
    # blockwise at the Llama-3-8B MLP up-projection
    "llama3_8b_mlp_block": _cfg(3, "llama3_8b_mlp_block", "block", 8192, 14336, 4096,
                                ("outliers", 1.0, 0.01, 50.0), ("normal", 0.02),
                                ("normal", 1e-4), gemms=("fprop", "dgrad", "wgrad")),
    # MXFP8 at the Llama-3-70B MLP
    "llama3_70b_mlp_mx": _cfg(4, "llama3_70b_mlp_mx", "mx", 16384, 28672, 8192,
                              ("outliers", 1.0, 0.005, 100.0), ("normal", 0.015),
                              ("normal", 1e-4), gemms=("fprop", "dgrad", "wgrad")),
    # one GPU's full Llama-3.1-405B MLP layer, blockwise
    "llama31_405b_mlp_block": _cfg(5, "llama31_405b_mlp_block", "block", 8192, 53248, 16384,
                                   ("gains", 1.0), ("normal", 0.01), ("normal", 1e-5),
                                   gemms=("fprop", "dgrad", "wgrad")),
}


def history_draw(cfg: Config, t: int, device: str = "cpu", rows: int | None = None) -> torch.Tensor:
    """Gradient draw t (seed history_seed0 + t) with G's shape and distribution;
    draws 0..history_draws-1 fill the amax history, draw history_draws is the
    gradient the timed step quantizes."""
    g = cfg.G
    return make(Tensor(g.name, g.rows, g.cols, g.kind, g.sigma, cfg.history_seed0 + t), device, rows)
