"""GPU parity of the FP8 linear layer (forward Y, backward dX and dW) against
the oracle composed the way each recipe prescribes.

The oracle quantizes the same BF16 inputs along the contraction dimension of
each GEMM (per-tensor recipes: one scale, the transposed operand is the same
codes transposed), dequantizes in float64 and contracts; every output entry
must satisfy |C - C_ref| <= 2^-10 sum|ab| + u_out |C_ref|.  Shapes span
several 256-wide GEMM tiles with ragged tails (272 tokens, 320 outputs)."""
import copy

import numpy as np
import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm
import oracle
import workloads
from fp8_scaled_quantization_scale_amd import linear as fl
from gpu_util import FMT_NAME, host, need_gpu

pytestmark = pytest.mark.gpu

B, T, K, N = 2, 136, 384, 320  # M = 272 tokens


def _inputs(seed, w_dtype=torch.bfloat16):
    x = workloads.make(workloads.Tensor("X", B * T, K, "outliers", 1.0, seed, 0.02, 50.0))
    w = workloads.make(workloads.Tensor("W", N, K, "normal", 0.02, seed + 1))
    g = workloads.make(workloads.Tensor("G", B * T, N, "normal", 1e-4, seed + 2))
    return x, w.to(w_dtype), g


class OracleRole:
    """Oracle side of one tensor role: dequantized operand with the
    contraction dimension last, for a given per-tensor scale or block recipe."""

    def __init__(self, rec, fmt):
        self.rec, self.fmt = rec, FMT_NAME[fmt]

    def deq(self, x, s=None, tiles=False):
        """x: float32 [rows x contraction]."""
        f = self.fmt
        if self.rec == fm.TENSOR_CURRENT:
            q, _, si, _, _ = oracle.quantize_current(f, x)
            return oracle.dequant(f, q, si)
        if self.rec == fm.TENSOR_DELAYED:
            q, _ = oracle.quantize_delayed(f, x, s)
            return oracle.dequant(f, q, np.float32(1.0) / np.float32(s))
        if self.rec == fm.CHANNEL:
            q, si, _ = oracle.quantize_channel(f, x)
            return oracle.dequant(f, q, si[:, None], 1, x.shape[1])
        if self.rec == fm.MX_1x32:
            q, g, _ = oracle.quantize_mx(f, x, 1, 32)
            return oracle.dequant_mx(f, q, g, 1, 32)
        br = 128 if tiles else 1
        q, g, _ = oracle.quantize_blocks(f, x, br, 128)
        return oracle.dequant(f, q, g, br, 128)


def _expect(p, x, w, g, scales=None):
    """Oracle Y, dX, dW for one step; scales = per-role delayed scales."""
    sc = scales or {}
    ox, ow, og = (OracleRole(*p.quant[r]) for r in ("x", "w", "g"))
    xf, wf, gf = x.float().numpy(), w.float().numpy(), g.float().numpy()
    per_tensor = p.quant["x"][0] in (fm.TENSOR_CURRENT, fm.TENSOR_DELAYED)
    tiles = p.quant["w"][0] == fm.BLOCK_128x128
    dx_ = ox.deq(xf, sc.get("x"))
    dw_ = ow.deq(wf, sc.get("w"), tiles)
    dg_ = og.deq(gf, sc.get("g"))
    if per_tensor:  # one scale per tensor: the transposed operands are the same values
        xt, wt, gt = dx_.T, dw_.T, dg_.T
    else:           # re-quantized along the other dimension
        xt = ox.deq(np.ascontiguousarray(xf.T))
        wt = ow.deq(np.ascontiguousarray(wf.T), None, tiles)
        gt = og.deq(np.ascontiguousarray(gf.T))
    return {"y": oracle.gemm_ref(dx_, dw_), "dx": oracle.gemm_ref(dg_, wt),
            "dw": oracle.gemm_ref(gt, xt)}


def _check(got, ref, out, tag):
    c_ref, s = ref
    bad = oracle.gemm_violations(host(got.detach().float()), c_ref, s, out)
    assert not bad.any(), (tag, int(bad.sum()), np.argwhere(bad)[:5])


def _step(lin, x, g):
    xd = x.cuda().reshape(B, T, K).requires_grad_(True)
    y = lin(xd)
    y.backward(g.cuda().reshape(B, T, N))
    torch.cuda.synchronize()
    return y.reshape(B * T, N), xd.grad.reshape(B * T, K), lin.weight.grad


RECIPES = {"current": fl.Float8CurrentScaling(), "block": fl.Float8BlockScaling(),
           "mx": fl.MXFP8BlockScaling(), "block_hybrid": fl.Float8BlockScaling(fl.Format.HYBRID),
           "mx_hybrid": fl.MXFP8BlockScaling(fl.Format.HYBRID), "channel": fl.Float8ChannelScaling(),
           "channel_hybrid": fl.Float8ChannelScaling(fl.Format.HYBRID)}


@pytest.mark.parametrize("name", list(RECIPES))
def test_linear_matches_oracle(name):
    need_gpu()
    r = RECIPES[name]
    x, w, g = _inputs(7100)
    lin = fl.Linear(K, N, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(w.cuda())
    with fl.fp8_autocast(fp8_recipe=r):
        y, dx, dw = _step(lin, x, g)
    ref = _expect(fl.plan(r), x, w, g)
    assert y.dtype == dx.dtype == dw.dtype == torch.bfloat16
    _check(y, ref["y"], "bf16", "y")
    _check(dx, ref["dx"], "bf16", "dx")
    _check(dw, ref["dw"], "bf16", "dw")


def test_linear_fp32_master_weight():
    """FP32 weight and input: FP32 GEMM outputs, held to the strict bound."""
    need_gpu()
    r = fl.Float8BlockScaling()
    x, w, g = _inputs(7200, torch.float32)
    x, g = x.float(), g.float()
    lin = fl.Linear(K, N, device="cuda", dtype=torch.float32, recipe=r)
    with torch.no_grad():
        lin.weight.copy_(w.cuda())
    y, dx, dw = _step(lin, x, g)
    assert y.dtype == dx.dtype == dw.dtype == torch.float32
    ref = _expect(fl.plan(r), x, w, g)
    _check(y, ref["y"], "fp32", "y")
    _check(dx, ref["dx"], "fp32", "dx")
    _check(dw, ref["dw"], "fp32", "dw")


def _history_scales(p, amaxes, length=200):
    """Oracle scales after pushing each role's amax sequence."""
    out = {}
    for role in ("x", "w", "g"):
        h = oracle.History(FMT_NAME[p.quant[role][1]], length)
        for a in amaxes[role]:
            h.update(a)
        out[role] = h.scale
    return out


def test_linear_delayed_two_steps_and_checkpoint():
    """Step 1 casts with the initial scale 1; step 2 with the scales the
    history derived from step 1's amax.  A module restored from the state
    after step 1 gives step 2 bit for bit."""
    need_gpu()
    r = fl.DelayedScaling()
    p = fl.plan(r)
    x1, w, g1 = _inputs(7300)
    x2, _, g2 = _inputs(7310)
    lin = fl.Linear(K, N, device="cuda", recipe=r)
    with torch.no_grad():
        lin.weight.copy_(w.cuda())
    y, dx, dw = _step(lin, x1, g1)
    ref = _expect(p, x1, w, g1, {"x": 1.0, "w": 1.0, "g": 1.0})
    for t, k in ((y, "y"), (dx, "dx"), (dw, "dw")):
        _check(t, ref[k], "bf16", "step1 " + k)

    saved = copy.deepcopy(lin.state_dict())
    lin.weight.grad = None
    y, dx, dw = _step(lin, x2, g2)
    am = {"x": [oracle.amax(x1.float().numpy())], "w": [oracle.amax(w.float().numpy())],
          "g": [oracle.amax(g1.float().numpy())]}
    sc = _history_scales(p, am)
    ref = _expect(p, x2, w, g2, sc)
    for t, k in ((y, "y"), (dx, "dx"), (dw, "dw")):
        _check(t, ref[k], "bf16", "step2 " + k)
    roles = lin._roles
    assert int(host(roles["x"].state.head)[0]) == 2 and int(host(roles["g"].state.head)[0]) == 2

    lin2 = fl.Linear(K, N, device="cuda", recipe=r)
    lin2.load_state_dict(saved)
    y2, dx2, dw2 = _step(lin2, x2, g2)
    assert torch.equal(y2, y) and torch.equal(dx2, dx) and torch.equal(dw2, dw)


def test_linear_delayed_interval():
    """interval=2: the history advances on every second cast of a role, and
    the scale in between stays the one derived before."""
    need_gpu()
    r = fl.DelayedScaling(interval=2)
    x1, w, g1 = _inputs(7400)
    x2, _, g2 = _inputs(7410)
    lin = fl.Linear(K, N, device="cuda", recipe=r)
    with torch.no_grad():
        lin.weight.copy_(w.cuda())
    _step(lin, x1, g1)
    st = lin._roles["x"].state
    assert int(host(st.head)[0]) == 0 and host(st.scale)[0] == np.float32(1.0)
    _step(lin, x2, g2)
    a = max(oracle.amax(x1.float().numpy()), oracle.amax(x2.float().numpy()))
    s, _, _ = oracle.scale_from_amax("e4m3", a)
    assert int(host(st.head)[0]) == 1 and host(st.history)[0] == np.float32(a)
    assert host(st.scale)[0] == s


def test_linear_inference_and_empty_batch():
    """Under no_grad only the ROW casts run; an empty batch gives an empty
    output and a zero weight gradient."""
    need_gpu()
    r = fl.Float8CurrentScaling()
    x, w, g = _inputs(7500)
    lin = fl.Linear(K, N, device="cuda", recipe=r)
    with torch.no_grad():
        lin.weight.copy_(w.cuda())
        y = lin(x.cuda())
    _check(y, _expect(fl.plan(r), x, w, g)["y"], "bf16", "y")
    xe = torch.empty(0, K, dtype=torch.bfloat16, device="cuda", requires_grad=True)
    ye = lin(xe)
    assert ye.shape == (0, N)
    ye.backward(torch.empty(0, N, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert xe.grad.shape == (0, K)
    assert not lin.weight.grad.float().abs().sum().item()
