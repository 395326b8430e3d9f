"""FP8 linear layer over the libfp8mi C ABI.

One ``nn.Linear``-shaped layer (weight stored [out x in], no bias) whose three
GEMMs -- fprop Y = X W^T, dgrad dX = dY W, wgrad dW = dY^T X -- take FP8
operands and keep a BF16/FP32 output, as "2025 technical guide: FP8 quantized
training" sec. 3.1 describes.  Every cast and every product runs in the HIP
library; torch only allocates, reshapes and drives autograd.  There is no
higher-precision path: without an FP8 recipe, on a CPU tensor, or without the
built library, the layer raises.

Recipes (the objects the guide's sec. 2.1-2.2 examples pass to
``fp8_autocast``, and "From FP16 to FP8" sec. 3.3's ``DelayedScaling``):

* ``DelayedScaling``  -- per-tensor scale taken from the largest amax of the
  last ``amax_history_len`` updates; a history update runs every ``interval``
  casts of a tensor role, the amax of the casts in between accumulating
  (guide sec. 2.1, "Mastering FP8 LLM training" strategy 1).
* ``Float8CurrentScaling`` -- per-tensor scale from the tensor's own amax
  (guide sec. 2.1, strategy 2).
* ``Float8BlockScaling`` -- 1x128 blocks for activations and gradients along
  the contraction dimension of each GEMM, 128x128 tiles for the weight (guide
  sec. 2.2); the wgrad operands are re-quantized along the token dimension
  (strategy 3).
* ``MXFP8BlockScaling`` -- 1x32 blocks with E8M0 scales for every operand
  along every contraction dimension (guide sec. 2.3, strategy 4).  The guide
  prints no class name for it; this one follows the other two.
* ``Float8ChannelScaling`` -- one scale per channel: per token row of X and
  dY, per output channel of W, and for each backward GEMM per channel of the
  transposed operand ("Mastering FP8 LLM training", Fig. 1 discussion of
  channel-wise scaling).  Name chosen here; the pages print none.

``Format.HYBRID`` puts activations and weights in E4M3 and gradients in E5M2
(guide sec. 2.1 hybrid format; "FP8 training support", "Why FP8?").  The
backward treats the casts as identity: gradients flow through the quantizer
unchanged (the straight-through estimator of "FP8 training support").
"""
from __future__ import annotations

import contextlib
import enum
import threading
from dataclasses import dataclass

import torch

from . import (BLOCK_1x128, BLOCK_128x128, CHANNEL, COL, E4M3, E5M2, GEMM_BLOCK_1x128_1x128,
               GEMM_BLOCK_1x128_128x128, GEMM_CHANNEL, GEMM_MX_1x32, GEMM_TENSOR, MX_1x32, ROW,
               TENSOR_CURRENT, TENSOR_DELAYED, DelayedState, Fp8Error, gemm, load, quantize)


class Format(enum.Enum):
    E4M3 = "E4M3"      # every tensor E4M3
    E5M2 = "E5M2"      # every tensor E5M2
    HYBRID = "HYBRID"  # activations and weights E4M3, gradients E5M2


@dataclass(frozen=True)
class DelayedScaling:
    margin: int = 0
    interval: int = 1
    fp8_format: Format = Format.HYBRID
    amax_history_len: int = 200


@dataclass(frozen=True)
class Float8CurrentScaling:
    fp8_format: Format = Format.HYBRID
    margin: int = 0


@dataclass(frozen=True)
class Float8BlockScaling:
    fp8_format: Format = Format.E4M3


@dataclass(frozen=True)
class MXFP8BlockScaling:
    fp8_format: Format = Format.E4M3


@dataclass(frozen=True)
class Float8ChannelScaling:
    fp8_format: Format = Format.E4M3
    margin: int = 0


RECIPES = (DelayedScaling, Float8CurrentScaling, Float8BlockScaling, MXFP8BlockScaling, Float8ChannelScaling)
ROLES = ("x", "w", "g")  # input activation, weight, output gradient


@dataclass(frozen=True)
class Plan:
    """What a recipe asks of the library: per tensor role the quantize recipe
    and format; per GEMM the scaled-GEMM recipe."""
    quant: dict   # role -> (quantize recipe, fmt)
    gemm: dict    # "fprop" / "dgrad" / "wgrad" -> GEMM recipe
    margin: int = 0


def _formats(f: Format):
    if f == Format.E4M3:
        return E4M3, E4M3
    if f == Format.E5M2:
        return E5M2, E5M2
    if f == Format.HYBRID:
        return E4M3, E5M2
    raise Fp8Error(f"unknown FP8 format {f!r}")


def plan(recipe) -> Plan:
    """Map a recipe object to library calls."""
    if not isinstance(recipe, RECIPES):
        raise Fp8Error(f"not an FP8 recipe: {recipe!r}")
    fwd, bwd = _formats(recipe.fp8_format)
    if isinstance(recipe, (DelayedScaling, Float8CurrentScaling)):
        if not 0 <= recipe.margin <= 64:
            raise Fp8Error("margin must be in [0, 64]")
        q = TENSOR_DELAYED if isinstance(recipe, DelayedScaling) else TENSOR_CURRENT
        if isinstance(recipe, DelayedScaling) and (recipe.interval < 1 or not 1 <= recipe.amax_history_len <= 65536):
            raise Fp8Error("interval must be >= 1 and amax_history_len in [1, 65536]")
        return Plan({"x": (q, fwd), "w": (q, fwd), "g": (q, bwd)},
                    {"fprop": GEMM_TENSOR, "dgrad": GEMM_TENSOR, "wgrad": GEMM_TENSOR}, recipe.margin)
    if isinstance(recipe, Float8ChannelScaling):
        if not 0 <= recipe.margin <= 64:
            raise Fp8Error("margin must be in [0, 64]")
        return Plan({"x": (CHANNEL, fwd), "w": (CHANNEL, fwd), "g": (CHANNEL, bwd)},
                    {"fprop": GEMM_CHANNEL, "dgrad": GEMM_CHANNEL, "wgrad": GEMM_CHANNEL}, recipe.margin)
    if isinstance(recipe, Float8BlockScaling):
        return Plan({"x": (BLOCK_1x128, fwd), "w": (BLOCK_128x128, fwd), "g": (BLOCK_1x128, bwd)},
                    {"fprop": GEMM_BLOCK_1x128_128x128, "dgrad": GEMM_BLOCK_1x128_128x128,
                     "wgrad": GEMM_BLOCK_1x128_1x128})
    return Plan({"x": (MX_1x32, fwd), "w": (MX_1x32, fwd), "g": (MX_1x32, bwd)},
                {"fprop": GEMM_MX_1x32, "dgrad": GEMM_MX_1x32, "wgrad": GEMM_MX_1x32})


# ---------------------------------------------------------------------------
# fp8_autocast: a thread-local recipe stack
# ---------------------------------------------------------------------------

_local = threading.local()


def _stack():
    if not hasattr(_local, "stack"):
        _local.stack = []
    return _local.stack


@contextlib.contextmanager
def fp8_autocast(enabled: bool = True, fp8_recipe=None):
    """Run ``Linear`` layers inside the block with ``fp8_recipe`` (default
    ``DelayedScaling()``).  ``enabled=False`` leaves the enclosing recipe (or
    each layer's own) in force."""
    if enabled:
        r = DelayedScaling() if fp8_recipe is None else fp8_recipe
        plan(r)  # reject a bad recipe on entry
        _stack().append(r)
    try:
        yield
    finally:
        if enabled:
            _stack().pop()


def active_recipe():
    s = _stack()
    return s[-1] if s else None


# ---------------------------------------------------------------------------
# the autograd function
# ---------------------------------------------------------------------------

def _scales(q, recipe: int, layout: int):
    """The GEMM-side scale tensor of one operand layout of a Quantized."""
    if recipe in (TENSOR_CURRENT, TENSOR_DELAYED):
        return q.scale_inv
    return q.s_row if layout == ROW else q.s_col


class _Role:
    """Per-role delayed-scaling state plus the cast counter that paces the
    history updates."""

    def __init__(self, fmt: int, length: int, margin: int, device):
        self.state = DelayedState(fmt, length, margin, device)
        self.casts = 0

    def cast(self, x2d: torch.Tensor, orient: int, interval: int):
        st = self.state
        q = quantize(x2d, TENSOR_DELAYED, st.fmt, orient, st.margin, scale=st.scale, amax=st.amax)
        q.scale_inv = st.scale_inv.clone()  # the pair this cast used; an update replaces it
        self.casts += 1
        if self.casts % interval == 0:
            st.update()
        return q


def _cast(role: str, x2d, orient, p: Plan, states, interval):
    rec, fmt = p.quant[role]
    if rec == TENSOR_DELAYED:
        return states[role].cast(x2d, orient, interval)
    return quantize(x2d, rec, fmt, orient, p.margin)


class _Fp8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2d, weight, p: Plan, states, interval, need_dx, need_dw):
        M, K = x2d.shape
        N = weight.shape[0]
        qx = _cast("x", x2d, ROW | (COL if need_dw else 0), p, states, interval)
        qw = _cast("w", weight, ROW | (COL if need_dx else 0), p, states, interval)
        rx, rw = p.quant["x"][0], p.quant["w"][0]
        y = gemm(qx.q_row, qx.fmt, _scales(qx, rx, ROW), qw.q_row, qw.fmt, _scales(qw, rw, ROW),
                 p.gemm["fprop"], K, torch.float32 if x2d.dtype == torch.float32 else torch.bfloat16,
                 M=M, N=N)
        # keep only what the backward GEMMs read: the transposed codes and their scales
        ctx.p, ctx.states, ctx.interval = p, states, interval
        ctx.need = (need_dx, need_dw)
        ctx.shape = (M, N, K)
        ctx.dtypes = (x2d.dtype, weight.dtype)
        ctx.fmts = (qx.fmt, qw.fmt)
        saved = []
        saved += [qx.q_col, _scales(qx, rx, COL)] if need_dw else [None, None]
        saved += [qw.q_col, _scales(qw, rw, COL)] if need_dx else [None, None]
        ctx.save_for_backward(*saved)
        return y

    @staticmethod
    def backward(ctx, dy):
        qxt, sxt, qwt, swt = ctx.saved_tensors
        p, states, interval = ctx.p, ctx.states, ctx.interval
        M, N, K = ctx.shape
        x_dt, w_dt = ctx.dtypes
        fx, fw = ctx.fmts
        need_dx, need_dw = ctx.need
        dy = dy.contiguous()
        if dy.dtype not in (torch.bfloat16, torch.float32):
            dy = dy.float()
        qg = _cast("g", dy, (ROW if need_dx else 0) | (COL if need_dw else 0), p, states, interval)
        rg = p.quant["g"][0]
        dx = dw = None
        if need_dx:  # dX[M x K] = dY[M x N] . (W^T)[K x N]^T
            dx = gemm(qg.q_row, qg.fmt, _scales(qg, rg, ROW), qwt, fw, swt, p.gemm["dgrad"], N,
                      torch.float32 if x_dt == torch.float32 else torch.bfloat16, M=M, N=K)
        if need_dw:  # dW[N x K] = (dY^T)[N x M] . (X^T)[K x M]^T
            dw = gemm(qg.q_col, qg.fmt, _scales(qg, rg, COL), qxt, fx, sxt, p.gemm["wgrad"], M,
                      torch.float32 if w_dt == torch.float32 else torch.bfloat16, M=N, N=K)
        return dx, dw, None, None, None, None, None


class Linear(torch.nn.Module):
    """y = x W^T with FP8 GEMMs.  ``weight`` is [out_features x in_features]
    (the nn.Linear layout), BF16 or FP32.  The recipe is the innermost
    ``fp8_autocast``'s, else the one given here; there is no other path.

    Sizes: in_features and out_features multiples of 16 (each is the
    contraction dimension of one GEMM); when the weight needs a gradient the
    token count (all leading dimensions of x together) is a multiple of 16 too
    (wgrad contracts over it)."""

    def __init__(self, in_features: int, out_features: int, bias: bool = False, recipe=None,
                 device=None, dtype=torch.bfloat16):
        super().__init__()
        if bias:
            raise Fp8Error("bias is not supported: the FP8 recipes cover the GEMM inputs only")
        if in_features % 16 or out_features % 16:
            raise Fp8Error("in_features and out_features must be multiples of 16")
        self.in_features, self.out_features = in_features, out_features
        self.recipe = recipe
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, device=device, dtype=dtype))
        torch.nn.init.kaiming_uniform_(self.weight, a=5 ** 0.5)
        self._roles: dict[str, _Role] = {}
        self._roles_key = None

    def _delayed_states(self, r: DelayedScaling, p: Plan, device):
        key = (r.fp8_format, r.amax_history_len, r.margin, str(device))
        if self._roles_key != key:
            self._roles = {role: _Role(p.quant[role][1], r.amax_history_len, r.margin, device) for role in ROLES}
            self._roles_key = key
        return self._roles

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        r = active_recipe() or self.recipe
        if r is None:
            raise Fp8Error("no FP8 recipe: pass recipe= or call inside fp8_autocast")
        p = plan(r)
        if not x.is_cuda or not self.weight.is_cuda:
            raise Fp8Error("the FP8 linear layer runs on the GPU only")
        if x.shape[-1] != self.in_features:
            raise Fp8Error(f"input has {x.shape[-1]} features, the layer {self.in_features}")
        if x.dtype not in (torch.bfloat16, torch.float32) or self.weight.dtype not in (torch.bfloat16, torch.float32):
            raise Fp8Error("inputs and weights are BF16 or FP32")
        load()
        lead = x.shape[:-1]
        x2d = x.reshape(-1, self.in_features).contiguous()
        grad = torch.is_grad_enabled()
        need_dx, need_dw = grad and x.requires_grad, grad and self.weight.requires_grad
        if need_dw and x2d.shape[0] % 16:
            raise Fp8Error("the token count must be a multiple of 16 when the weight needs a gradient")
        states = self._delayed_states(r, p, x.device) if isinstance(r, DelayedScaling) else None
        interval = r.interval if isinstance(r, DelayedScaling) else 1
        y = _Fp8LinearFn.apply(x2d, self.weight.contiguous(), p, states, interval, need_dx, need_dw)
        return y.reshape(*lead, self.out_features)

    # delayed-scaling state travels with the module's state_dict
    def get_extra_state(self):
        return {"key": self._roles_key,
                "roles": {k: {"casts": v.casts, "fmt": v.state.fmt, "margin": v.state.margin,
                              "tensors": v.state.state_dict()} for k, v in self._roles.items()}}

    def set_extra_state(self, state):
        if not state or not state.get("roles"):
            return
        roles = {}
        for role, sd in state["roles"].items():
            t = sd["tensors"]
            r = _Role(sd["fmt"], t["history"].numel(), sd["margin"], t["history"].device)
            r.casts = int(sd["casts"])
            r.state.load_state_dict(t)
            roles[role] = r
        self._roles, self._roles_key = roles, state["key"]
