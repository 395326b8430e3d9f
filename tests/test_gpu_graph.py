"""The library allocates nothing, keeps no host state and records no memset,
so a whole step of the path can be captured in a HIP graph and replayed.
One step of the per-tensor workload at reduced size (current-scaling casts
of X and W, the delayed cast of G, fprop, dgrad, the amax-history update)
is captured once and replayed several times, with eager work and
synchronisations between the replays; every replay must equal, bit for bit,
the same step run eagerly from the same state on the same inputs (codes,
scales, GEMM outputs and the delayed-scaling state it advances)."""
import pytest
import torch

import fp8_scaled_quantization_scale_amd as fm
import workloads
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

M, N, K = 1024, 768, 512


class StepBuffers:
    """Inputs, outputs and delayed state of one step, at fixed addresses."""

    def __init__(self):
        d = "cuda"
        u8 = torch.uint8
        self.X = torch.empty(M, K, dtype=torch.bfloat16, device=d)
        self.W = torch.empty(N, K, dtype=torch.bfloat16, device=d)
        self.G = torch.empty(M, N, dtype=torch.bfloat16, device=d)
        self.qx, self.qw, self.qwt, self.qg = (torch.empty(M, K, dtype=u8, device=d), torch.empty(N, K, dtype=u8, device=d),
                                               torch.empty(K, N, dtype=u8, device=d), torch.empty(M, N, dtype=u8, device=d))
        f = lambda n=1: torch.zeros(n, dtype=torch.float32, device=d)  # noqa: E731
        self.sx, self.six, self.ax = f(), f(), f(fm.AMAX_SLOTS)
        self.sw, self.siw, self.aw = f(), f(), f(fm.AMAX_SLOTS)
        self.state = fm.DelayedState(fm.E5M2, 200, 0, d)
        self.y = torch.empty(M, N, dtype=torch.bfloat16, device=d)
        self.dx = torch.empty(M, K, dtype=torch.bfloat16, device=d)

    def step(self):
        st = self.state
        ok = lambda s: fm._check(s, "step")  # noqa: E731
        ok(fm.fp8_quantize(self.X, fm.IN_BF16, M, K, K, fm.TENSOR_CURRENT, fm.E4M3, fm.ROW, 0,
                           self.qx, K, None, None, 0, None, self.sx, self.six, self.ax, None))
        ok(fm.fp8_quantize(self.W, fm.IN_BF16, N, K, K, fm.TENSOR_CURRENT, fm.E4M3, fm.ROW_AND_COL, 0,
                           self.qw, K, None, self.qwt, N, None, self.sw, self.siw, self.aw, None))
        ok(fm.fp8_quantize(self.G, fm.IN_BF16, M, N, N, fm.TENSOR_DELAYED, fm.E5M2, fm.ROW, 0,
                           self.qg, N, None, None, 0, None, st.scale, None, st.amax, st.nonfinite))
        ok(fm.fp8_gemm_scaled(self.qx, fm.E4M3, self.six, K, self.qw, fm.E4M3, self.siw, K,
                              fm.GEMM_TENSOR, fm.LAYOUT_TN, M, N, K, self.y, fm.OUT_BF16, N))
        ok(fm.fp8_gemm_scaled(self.qg, fm.E5M2, st.scale_inv, N, self.qwt, fm.E4M3, self.siw, N,
                              fm.GEMM_TENSOR, fm.LAYOUT_TN, M, K, N, self.dx, fm.OUT_BF16, K))
        ok(fm.fp8_amax_history_update(st.history, st.head, 200, st.amax, fm.E5M2, 0,
                                      st.scale, st.scale_inv, st.nonfinite))

    def load(self, x, w, g, state_sd):
        self.X.copy_(x)
        self.W.copy_(w)
        self.G.copy_(g)
        self.state.load_state_dict(state_sd)

    def results(self):
        out = {k: getattr(self, k).clone() for k in ("qx", "qw", "qwt", "qg", "sx", "six", "ax", "sw", "siw",
                                                       "y", "dx")}
        out["ax"] = out["ax"][:1]
        out["aw"] = self.aw[:1].clone()
        out.update({"state_" + k: v for k, v in self.state.state_dict().items()})
        return out


def _inputs(r):
    c = workloads.CONFIGS["llama3_8b_attn_tensor"]
    mk = lambda t, rows, cols, seed: workloads.make(  # noqa: E731
        workloads.Tensor(t.name, rows, cols, t.kind, t.sigma, seed, t.frac, t.factor), "cuda")
    return (mk(c.X, M, K, 9100 + r), mk(c.W, N, K, 9200 + r), mk(c.G, M, N, 9300 + r))


def _same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def test_step_graph_replays_match_eager():
    need_gpu()
    eager, graphed = StepBuffers(), StepBuffers()
    # a history with some content, the same for both
    for t in range(5):
        x, w, g = _inputs(10 + t)
        eager.X.copy_(x)
        eager.W.copy_(w)
        eager.G.copy_(g)
        eager.step()
    sd = eager.state.state_dict()

    # capture (after a warm-up launch of every kernel on this side stream)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graphed.load(*_inputs(0), sd)
        graphed.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.step()
    torch.cuda.synchronize()

    state = sd
    for r in range(1, 5):
        x, w, g = _inputs(r)
        eager.load(x, w, g, state)
        eager.step()
        want = eager.results()
        torch.cuda.synchronize()
        graphed.load(x, w, g, state)
        graph.replay()
        torch.cuda.synchronize()
        got = graphed.results()
        for k in want:
            assert _same(got[k], want[k]), (r, k)
        state = {k[len("state_"):]: v for k, v in want.items() if k.startswith("state_")}
        # eager work between replays on the same buffers
        graphed.step()
        torch.cuda.synchronize()
