"""GPU parity of the delayed-scaling step (fp8_quantize with TENSOR_DELAYED +
fp8_amax_history_update) against the oracle's History over 450 steps: ring,
head, scale, scale_inv and the non-finite counter bit for bit, including the
step where the first amax leaves the 200-entry window, and a save/restore in
the middle of the run."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm
import oracle
import workloads
from gpu_util import acc_amax, host, need_gpu, same_f32

pytestmark = pytest.mark.gpu


def _run(state: fm.DelayedState, ref: oracle.History, draws, check_every=1):
    for t, x in enumerate(draws):
        q = state.quantize(x, fm.ROW)
        oq, am = oracle.quantize_delayed(ref.fmt, x.float().cpu().numpy(), ref.scale)
        if t % check_every == 0:
            assert np.array_equal(host(q.q_row)[:, : x.shape[1]], oq), t
            assert same_f32([acc_amax(state.amax)], [am]), t
        state.update()
        if t % check_every == 0:
            assert not host(state.amax).view(np.uint32).any(), t
        ref.update(am)
        if t % check_every == 0:
            assert same_f32(host(state.scale), [ref.scale]), t
            assert same_f32(host(state.scale_inv), [ref.scale_inv]), t
    assert np.array_equal(host(state.history), ref.ring)
    assert host(state.head)[0] == ref.head[0]
    assert host(state.nonfinite)[0] == ref.nonfinite[0]


def test_history_450_steps_with_window_edge():
    need_gpu()
    g = torch.Generator().manual_seed(7)
    # amax decreasing over the first 220 steps so the window edge at 200 shows
    draws = []
    for t in range(450):
        x = torch.randn(64, 256, generator=g) * (1e-4 * (1.0 - 0.002 * min(t, 220)))
        draws.append(x.to(torch.bfloat16).cuda())
    draws[37][3, 3] = float("nan")
    draws[301][0, 0] = float("inf")
    state = fm.DelayedState(fm.E5M2, 200)
    ref = oracle.History("e5m2", 200)
    _run(state, ref, draws)


def test_history_save_restore_is_bit_identical():
    need_gpu()
    g = torch.Generator().manual_seed(8)
    draws = [(torch.randn(32, 128, generator=g) * 10 ** float(torch.empty(1).uniform_(-5, -3, generator=g)))
             .to(torch.bfloat16).cuda() for _ in range(400)]
    a = fm.DelayedState(fm.E5M2, 200)
    for x in draws:
        a.quantize(x)
        a.update()
    b = fm.DelayedState(fm.E5M2, 200)
    for x in draws[:200]:
        b.quantize(x)
        b.update()
    saved = {k: v.cpu() for k, v in b.state_dict().items()}
    c = fm.DelayedState(fm.E5M2, 200)
    c.load_state_dict({k: v.cuda() for k, v in saved.items()})
    for x in draws[200:]:
        c.quantize(x)
        c.update()
    for k in ("history", "head", "scale", "scale_inv", "amax", "nonfinite"):
        assert torch.equal(getattr(a, k), getattr(c, k)), k


def test_history_fill_from_seeded_draws_e4m3_margin():
    """E4M3 with margin 1 and a short ring, gradient draws of the attention
    projection's distribution (N(0, 1e-4))."""
    need_gpu()
    cfg = workloads.CONFIGS["llama3_8b_attn_tensor"]
    state = fm.DelayedState(fm.E4M3, 16, margin=1)
    ref = oracle.History("e4m3", 16, margin=1)
    draws = [workloads.history_draw(cfg, t, rows=64).cuda() for t in range(40)]
    _run(state, ref, draws)
