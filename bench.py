"""Benchmark of the FP8 training hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole path over one batch of synthetic inputs:
quantize every GEMM operand with the workload's recipe (including the
transposed layouts the backward GEMMs read), the delayed-scaling history
update where the recipe has one, then the fprop / dgrad (/ wgrad) scaled FP8
GEMMs.  The default workload is one GPU's full Llama-3.1-405B MLP layer in
the blockwise recipe (X 8192 x 16384, W 53248 x 16384, G 8192 x 53248;
transpose-quantize inside the timing).  Inputs are resident in HBM before
timing starts; R rotating copies of every input (default 4) keep each step's
reads from being served by the previous step's Infinity Cache contents.

Prints ONE JSON line.  `value` is GEMM FLOP of the step / step time (TFLOP/s),
so quantization time counts against it.
  * "roofline": the dominant GEMM (largest share of the step), timed inside
    the timed steps with HIP events on the stream it runs on, in every E-th
    step (--event-every); "roofline_fprop" the same for the fprop GEMM, the
    blockwise kernel the method's throughput target names.  Each carries the
    fraction of the 5.0 PFLOP/s datasheet peak and of the rates the matrix
    cores sustain on this GPU under full FP8 load ("mfma_ceiling", measured
    by libfp8mi_probe.so together with the shader clock under that load):
    with fixed operands (the clock limit) and with operands that change
    from product to product as a GEMM's do ("varied", the power limit).
  * "kernels": each op alone over back-to-back launches; casts report GB/s
    against the 8 TB/s datasheet figure and against "hbm_ceiling", in-tree
    streaming kernels at the cast's own read:write byte mix.
  * "event_pair_empty_us": what one pair of (fence-free) event records costs
    the queue, measured on an empty stretch of it.
  * "cpu_baseline": the CPU oracle timed on a bounded sample of the step and
    extrapolated to the full step (rank 0), on one thread and on every core.
`--workload tiny_block` (a parity-size case) prints a latency line instead:
microseconds per step (quantize A 1x128, quantize B 128x128, fprop GEMM),
launched eagerly and as a replayed HIP graph.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_scaled_quantization_scale_amd as fm  # noqa: E402
from fp8_scaled_quantization_scale_amd import probe  # noqa: E402
import workloads  # noqa: E402

PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, GB/s
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 / MXFP8 matrix peak, TFLOP/s
PEAK_CLOCK_GHZ = 2.4          # the clock the datasheet peak assumes
DEFAULT_WORKLOAD = "llama31_405b_mlp_block"


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------

class Step:
    """Device buffers and the launch sequence of one workload's step."""

    def __init__(self, cfg: workloads.Config, rotate: int):
        self.cfg = cfg
        M, N, K = cfg.M, cfg.N, cfg.K
        dev = "cuda"
        self.rotate = rotate
        # R copies of the inputs: copy r is the seeded draw with seed + 100 r
        self.X = [workloads.make(_reseed(cfg.X, r), dev) for r in range(rotate)]
        self.W = [workloads.make(_reseed(cfg.W, r), dev) for r in range(rotate)]
        self.G = [workloads.make(_reseed(cfg.G, r), dev) for r in range(rotate)]
        self.ops = []  # (name, kind, work, fn) with kind in {"quant", "gemm", "small"}
        rec = cfg.recipe
        self.outputs = {}
        if rec == "tensor":
            self._build_tensor()
        elif rec == "block":
            self._build_block()
        else:
            self._build_mx()

    # per-tensor hybrid: E4M3 X, W (current), E5M2 G (delayed, 200-step history)
    def _build_tensor(self):
        cfg = self.cfg
        M, N, K = cfg.M, cfg.N, cfg.K
        d = "cuda"
        u8 = torch.uint8
        self.qx = torch.empty(M, K, dtype=u8, device=d)
        self.qw = torch.empty(N, K, dtype=u8, device=d)
        self.qwt = torch.empty(K, N, dtype=u8, device=d)
        self.qg = torch.empty(M, N, dtype=u8, device=d)
        f = lambda n=1: torch.zeros(n, dtype=torch.float32, device=d)  # noqa: E731
        self.sx, self.six, self.ax = f(), f(), f(fm.AMAX_SLOTS)
        self.sw, self.siw, self.aw = f(), f(), f(fm.AMAX_SLOTS)
        self.state = fm.DelayedState(fm.E5M2, 200, 0, d)
        self.y = torch.empty(M, N, dtype=torch.bfloat16, device=d)
        self.dx = torch.empty(M, K, dtype=torch.bfloat16, device=d)
        # fill the amax history from 200 seeded gradient draws, then arm draw 200
        for t in range(cfg.history_draws):
            g = workloads.history_draw(cfg, t, d)
            fm.quantize(g, fm.TENSOR_DELAYED, fm.E5M2, fm.ROW, scale=self.state.scale,
                        amax=self.state.amax)
            self.state.update()
        self.G = [workloads.history_draw(cfg, cfg.history_draws + r, d) for r in range(self.rotate)]
        st = self.state

        def qx(r):
            x = self.X[r]
            _ok(fm.fp8_quantize(x, fm.IN_BF16, M, K, K, fm.TENSOR_CURRENT, fm.E4M3, fm.ROW, 0,
                                self.qx, K, None, None, 0, None, self.sx, self.six, self.ax, None))

        def qw(r):
            w = self.W[r]
            _ok(fm.fp8_quantize(w, fm.IN_BF16, N, K, K, fm.TENSOR_CURRENT, fm.E4M3, fm.ROW_AND_COL, 0,
                                self.qw, K, None, self.qwt, N, None, self.sw, self.siw, self.aw, None))

        def qg(r):
            g = self.G[r]
            _ok(fm.fp8_quantize(g, fm.IN_BF16, M, N, N, fm.TENSOR_DELAYED, fm.E5M2, fm.ROW, 0,
                                self.qg, N, None, None, 0, None, st.scale, None, st.amax, None))

        def hist(r):
            _ok(fm.fp8_amax_history_update(st.history, st.head, 200, st.amax, fm.E5M2, 0,
                                           st.scale, st.scale_inv, st.nonfinite))

        def fprop(r):
            _ok(fm.fp8_gemm_scaled(self.qx, fm.E4M3, self.six, K, self.qw, fm.E4M3, self.siw, K,
                                   fm.GEMM_TENSOR, fm.LAYOUT_TN, M, N, K, self.y, fm.OUT_BF16, N))

        def dgrad(r):
            # dX[M x K] = dY[M x N] . W[N x K]: A = dY codes, B = W^T codes [K x N]
            _ok(fm.fp8_gemm_scaled(self.qg, fm.E5M2, st.scale_inv, N, self.qwt, fm.E4M3, self.siw, N,
                                   fm.GEMM_TENSOR, fm.LAYOUT_TN, M, K, N, self.dx, fm.OUT_BF16, K))

        # the history update closes the step: dgrad must dequantize G's codes
        # with the scale_inv they were cast with, and the update replaces it
        # by the next step's
        self.ops = [
            ("quant_x_current_e4m3", "quant", M * K * 3, qx),
            ("quant_w_current_e4m3_row_col", "quant", N * K * 4, qw),
            ("quant_g_delayed_e5m2", "quant", M * N * 3, qg),
            ("gemm_fprop", "gemm", 2 * M * N * K, fprop),
            ("gemm_dgrad", "gemm", 2 * M * N * K, dgrad),
            ("history_update", "small", 0, hist),
        ]

    def _build_block(self):
        cfg = self.cfg
        M, N, K = cfg.M, cfg.N, cfg.K
        d = "cuda"
        u8, f32 = torch.uint8, torch.float32
        c = lambda a, b: (a + b - 1) // b  # noqa: E731
        self.qx, self.sx = torch.empty(M, K, dtype=u8, device=d), torch.empty(M, c(K, 128), dtype=f32, device=d)
        self.qxt, self.sxt = torch.empty(K, M, dtype=u8, device=d), torch.empty(K, c(M, 128), dtype=f32, device=d)
        self.qw, self.sw = torch.empty(N, K, dtype=u8, device=d), torch.empty(c(N, 128), c(K, 128), dtype=f32, device=d)
        self.qwt, self.swt = torch.empty(K, N, dtype=u8, device=d), torch.empty(c(K, 128), c(N, 128), dtype=f32, device=d)
        self.qg, self.sg = torch.empty(M, N, dtype=u8, device=d), torch.empty(M, c(N, 128), dtype=f32, device=d)
        self.qgt, self.sgt = torch.empty(N, M, dtype=u8, device=d), torch.empty(N, c(M, 128), dtype=f32, device=d)
        self.y = torch.empty(M, N, dtype=torch.bfloat16, device=d)
        self.dx = torch.empty(M, K, dtype=torch.bfloat16, device=d)
        self.dw = torch.empty(N, K, dtype=torch.bfloat16, device=d)

        def qx(r):
            _ok(fm.fp8_quantize(self.X[r], fm.IN_BF16, M, K, K, fm.BLOCK_1x128, fm.E4M3, fm.ROW_AND_COL, 0,
                                self.qx, K, self.sx, self.qxt, M, self.sxt, None, None, None, None))

        def qw(r):
            _ok(fm.fp8_quantize(self.W[r], fm.IN_BF16, N, K, K, fm.BLOCK_128x128, fm.E4M3, fm.ROW_AND_COL, 0,
                                self.qw, K, self.sw, self.qwt, N, self.swt, None, None, None, None))

        def qg(r):
            _ok(fm.fp8_quantize(self.G[r], fm.IN_BF16, M, N, N, fm.BLOCK_1x128, fm.E4M3, fm.ROW_AND_COL, 0,
                                self.qg, N, self.sg, self.qgt, M, self.sgt, None, None, None, None))

        def fprop(r):
            _ok(fm.fp8_gemm_scaled(self.qx, fm.E4M3, self.sx, K, self.qw, fm.E4M3, self.sw, K,
                                   fm.GEMM_BLOCK_1x128_128x128, fm.LAYOUT_TN, M, N, K, self.y, fm.OUT_BF16, N))

        def dgrad(r):
            _ok(fm.fp8_gemm_scaled(self.qg, fm.E4M3, self.sg, N, self.qwt, fm.E4M3, self.swt, N,
                                   fm.GEMM_BLOCK_1x128_128x128, fm.LAYOUT_TN, M, K, N, self.dx, fm.OUT_BF16, K))

        def wgrad(r):
            # dW[N x K] = dY^T[N x M] . X[M x K]: both operands blocked along M
            _ok(fm.fp8_gemm_scaled(self.qgt, fm.E4M3, self.sgt, M, self.qxt, fm.E4M3, self.sxt, M,
                                   fm.GEMM_BLOCK_1x128_1x128, fm.LAYOUT_TN, N, K, M, self.dw, fm.OUT_BF16, K))

        sc = 4 / 128
        self.ops = [
            ("quant_x_1x128_row_col", "quant", int(M * K * (2 + 1 + 1 + 2 * sc)), qx),
            ("quant_w_128x128_row_col", "quant", int(N * K * (2 + 1 + 1) + 2 * 4 * c(N, 128) * c(K, 128)), qw),
            ("quant_g_1x128_row_col", "quant", int(M * N * (2 + 1 + 1 + 2 * sc)), qg),
            ("gemm_fprop", "gemm", 2 * M * N * K, fprop),
            ("gemm_dgrad", "gemm", 2 * M * N * K, dgrad),
            ("gemm_wgrad", "gemm", 2 * M * N * K, wgrad),
        ]

    def _build_mx(self):
        cfg = self.cfg
        M, N, K = cfg.M, cfg.N, cfg.K
        d = "cuda"
        u8 = torch.uint8
        c = lambda a, b: (a + b - 1) // b  # noqa: E731
        e = lambda r, k: torch.empty(r, c(k, 32), dtype=u8, device=d)  # noqa: E731
        self.qx, self.sx = torch.empty(M, K, dtype=u8, device=d), e(M, K)
        self.qxt, self.sxt = torch.empty(K, M, dtype=u8, device=d), e(K, M)
        self.qw, self.sw = torch.empty(N, K, dtype=u8, device=d), e(N, K)
        self.qwt, self.swt = torch.empty(K, N, dtype=u8, device=d), e(K, N)
        self.qg, self.sg = torch.empty(M, N, dtype=u8, device=d), e(M, N)
        self.qgt, self.sgt = torch.empty(N, M, dtype=u8, device=d), e(N, M)
        self.y = torch.empty(M, N, dtype=torch.bfloat16, device=d)
        self.dx = torch.empty(M, K, dtype=torch.bfloat16, device=d)
        self.dw = torch.empty(N, K, dtype=torch.bfloat16, device=d)

        def q(src, rows, cols, qr, sr, qc, sc_):
            _ok(fm.fp8_quantize(src, fm.IN_BF16, rows, cols, cols, fm.MX_1x32, fm.E4M3, fm.ROW_AND_COL, 0,
                                qr, cols, sr, qc, rows, sc_, None, None, None, None))

        def fprop(r):
            _ok(fm.fp8_gemm_scaled(self.qx, fm.E4M3, self.sx, K, self.qw, fm.E4M3, self.sw, K,
                                   fm.GEMM_MX_1x32, fm.LAYOUT_TN, M, N, K, self.y, fm.OUT_BF16, N))

        def dgrad(r):
            _ok(fm.fp8_gemm_scaled(self.qg, fm.E4M3, self.sg, N, self.qwt, fm.E4M3, self.swt, N,
                                   fm.GEMM_MX_1x32, fm.LAYOUT_TN, M, K, N, self.dx, fm.OUT_BF16, K))

        def wgrad(r):
            _ok(fm.fp8_gemm_scaled(self.qgt, fm.E4M3, self.sgt, M, self.qxt, fm.E4M3, self.sxt, M,
                                   fm.GEMM_MX_1x32, fm.LAYOUT_TN, N, K, M, self.dw, fm.OUT_BF16, K))

        b = 2 + 1 + 1 + 2 / 32
        self.ops = [
            ("quant_x_mx_row_col", "quant", int(M * K * b),
             lambda r: q(self.X[r], M, K, self.qx, self.sx, self.qxt, self.sxt)),
            ("quant_w_mx_row_col", "quant", int(N * K * b),
             lambda r: q(self.W[r], N, K, self.qw, self.sw, self.qwt, self.swt)),
            ("quant_g_mx_row_col", "quant", int(M * N * b),
             lambda r: q(self.G[r], M, N, self.qg, self.sg, self.qgt, self.sgt)),
            ("gemm_fprop", "gemm", 2 * M * N * K, fprop),
            ("gemm_dgrad", "gemm", 2 * M * N * K, dgrad),
            ("gemm_wgrad", "gemm", 2 * M * N * K, wgrad),
        ]

    def run(self, r: int, timed_op: int = -1, events=None, pair: int = 0):
        """One step on input copy r; event pair `pair` brackets op `timed_op`."""
        for i, (_, _, _, fn) in enumerate(self.ops):
            if i == timed_op:
                events.record(pair, False)
            fn(r % self.rotate)
            if i == timed_op:
                events.record(pair, True)

    def gemm_flops(self) -> int:
        return sum(w for _, k, w, _ in self.ops if k == "gemm")


class HipEvents:
    """n pairs of HIP timing events created with hipEventDisableSystemFence,
    recorded on torch's current stream (the stream every op launches on).
    Bound to the HIP runtime torch has already loaded."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int = 1):
        hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
        vp = ctypes.c_void_p
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [vp, vp]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        hip.hipEventDestroy.argtypes = [vp]
        self.hip = hip
        self.pairs = [(self._new(), self._new()) for _ in range(n)]

    def _new(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def record(self, i: int, end: bool):
        e = self.pairs[i][1 if end else 0]
        if self.hip.hipEventRecord(e, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i: int) -> float:
        """Elapsed ms of pair i (both events recorded and complete)."""
        f = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(f), *self.pairs[i]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def __del__(self):
        for pair in getattr(self, "pairs", []):
            for e in pair:
                self.hip.hipEventDestroy(e)


def _reseed(t: workloads.Tensor, r: int) -> workloads.Tensor:
    return workloads.Tensor(t.name, t.rows, t.cols, t.kind, t.sigma, t.seed + 100 * r, t.frac, t.factor)


def _ok(status: int):
    if status != fm.OK:
        raise fm.Fp8Error(f"status {status}: {fm.status_string(status)}")


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample
# ---------------------------------------------------------------------------

def _threads() -> int:
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)


def cpu_baseline(cfg: workloads.Config, rows: int = 1024, out_rows: int = 768):
    """Time the oracle on a bounded sample of the step and extrapolate to the
    full step.  Quantize: `rows` whole rows of X, G and W (their codes and
    scales in every layout the step writes), cost scaled by M / rows (X, G)
    and N / rows (W).  GEMMs: an out_rows x out_rows block of each GEMM's
    output from oracle-quantized operand rows of that GEMM's contraction
    length (dequantize, float64 product), cost scaled by the output count.
    Timed on one thread, then with the quantize rows split over every core
    and the float64 products on every BLAS thread."""
    from concurrent.futures import ThreadPoolExecutor

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle

    M, N, K = cfg.M, cfg.N, cfg.K
    draw = lambda t, r, cols=None: workloads.make(  # noqa: E731
        t if cols is None else workloads.Tensor(t.name, r, cols, t.kind, t.sigma, t.seed, t.frac, t.factor),
        rows=r).float().numpy()
    x, g, w = draw(cfg.X, rows), draw(cfg.G, rows), draw(cfg.W, rows)
    rec = cfg.recipe

    def q_rows(v, br, bc):
        if rec == "mx":
            return oracle.quantize_mx("e4m3", v, br, bc)
        return oracle.quantize_blocks("e4m3", v, br, bc)

    def deq(q, gr, br, bc):
        if rec == "mx":
            return oracle.dequant_mx("e4m3", q, gr, br, bc)
        return oracle.dequant("e4m3", q, gr, br, bc)

    # layouts written per tensor: (tensor rows, its full row count, how)
    if rec == "tensor":
        jobs = [(x, M, "current"), (w, N, "current_t"), (g, M, "delayed")]
    elif rec == "block":
        jobs = [(x, M, (1, 128)), (x, M, (128, 1)), (w, N, (128, 128)), (w, N, "t128"), (g, M, (1, 128)),
                (g, M, (128, 1))]
    else:
        jobs = [(v, full, bl) for v, full in ((x, M), (w, N), (g, M)) for bl in ((1, 32), (32, 1))]

    def quant_job(v, how):
        if how == "current":
            oracle.quantize_current("e4m3", v)
        elif how == "current_t":
            q = oracle.quantize_current("e4m3", v)[0]
            np.ascontiguousarray(q.T)
        elif how == "delayed":
            oracle.quantize_delayed("e5m2", v, 1.0)
        elif how == "t128":
            q_rows(np.ascontiguousarray(v.T), 128, 128)
        else:
            q_rows(v, *how)

    def quant_parallel(ex, v, how, n):
        """Column chunks of whole blocks on n threads (per-tensor current
        scaling needs the whole tensor's amax first: one thread)."""
        if how in ("current", "current_t"):
            quant_job(v, how)
            return
        cols = v.shape[1]
        step = -(-cols // n // 128) * 128
        parts = [np.ascontiguousarray(v[:, c0:c0 + step]) for c0 in range(0, cols, step)]
        list(ex.map(lambda p: quant_job(p, how), parts))

    def gemm_operands(kc, ta, tb):
        """oracle-quantized, dequantized operand rows with contraction kc"""
        a = draw(ta, out_rows, kc)
        b = draw(tb, out_rows, kc)
        if rec == "tensor":
            qa, _, sa, _, _ = oracle.quantize_current("e4m3", a)
            qb, _, sb, _, _ = oracle.quantize_current("e4m3", b)
            return oracle.dequant("e4m3", qa, sa), oracle.dequant("e4m3", qb, sb)
        bl = (1, 32) if rec == "mx" else (1, 128)
        qa, ga, _ = q_rows(a, *bl)
        qb, gb, _ = q_rows(b, *bl)
        return deq(qa, ga, *bl), deq(qb, gb, *bl)

    shapes = {"fprop": (M, N, K, cfg.X, cfg.W), "dgrad": (M, K, N, cfg.G, cfg.W),
              "wgrad": (N, K, M, cfg.G, cfg.X)}

    def run(parallel: bool):
        """(quantize seconds, GEMM seconds, wall seconds of the sample), the
        first two extrapolated to the full step"""
        t0 = time.perf_counter()
        tq = 0.0
        with ThreadPoolExecutor(_threads()) as ex:
            for v, full, how in jobs:
                t1 = time.perf_counter()
                if parallel:
                    quant_parallel(ex, v, how, _threads())
                else:
                    quant_job(v, how)
                tq += (time.perf_counter() - t1) * full / v.shape[0]
        tg = 0.0
        for name in cfg.gemms:
            m, n, kc, ta, tb = shapes[name]
            da, db = gemm_operands(kc, ta, tb)
            t1 = time.perf_counter()
            oracle.gemm_ref(da, db)
            tg += (time.perf_counter() - t1) * (m * n) / (out_rows * out_rows)
        return tq, tg, time.perf_counter() - t0

    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx is not None:
        ctx.__enter__()
    try:
        q1, g1, wall1 = run(False)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    qa, ga, walla = run(True)
    flops = len(cfg.gemms) * 2.0 * M * N * K
    full1, fulla = q1 + g1, qa + ga
    return {
        "value": round(flops / full1 / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"oracle quantize of {rows} whole rows of X, G and W in every layout of the step and an "
                   f"{out_rows}x{out_rows} block of each GEMM's output (float64), on one thread; measured "
                   f"{wall1:.1f} s, extrapolated to the full step ({full1:.1f} s: quantize {q1:.1f} s scaled "
                   f"by rows, GEMMs {g1:.1f} s scaled by output count)"),
        "all_cores": {"value": round(flops / fulla / 1e12, 6), "cores": _threads(),
                      "note": f"same sample, quantize split by column blocks over {_threads()} threads, float64 products on "
                              f"every BLAS thread; measured {walla:.1f} s, extrapolated {fulla:.1f} s"},
        "host_cpu": _cpu_model(),
        "host_cpus_visible": _threads(),
    }


def _cpu_model() -> str:
    """Model name of the host CPU the baseline ran on (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------

def _source_sha() -> str:
    """Hash of the sources that define the path's kernels and their launch
    configuration (the HIP files and the two internal headers; not the C
    ABI's host-side validation in api.cpp, which does not change what a
    kernel moves, nor the measurement kernels of probe.hip), comments and
    blank space left out so that an edited comment does not orphan the
    counters taken on the same code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_scaled_quantization_scale_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if (f.endswith(".hip") and f != "probe.hip") or f in ("device.hpp", "launch.hpp"):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                text = fh.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # (no string literal in these holds // or /*)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_sha") != _source_sha():
        return None
    return ent.get("bytes_per_launch")


CEIL_BYTES = 1 << 30  # source bytes of each ceiling stream (4x the Infinity Cache)
MIX_OF = {"ROW": probe.HALF, "ROW_AND_COL": probe.SPLIT, "COPY": probe.COPY, "READ": probe.READ}


def hbm_ceilings(ev: "HipEvents") -> dict:
    """GB/s this GPU sustains for plain in-tree streams (libfp8mi_probe.so)
    at each read:write byte mix: READ, COPY (1:1), ROW (2 bytes in, 1 out: a
    cast writing one code layout) and ROW_AND_COL (2 in, 1 + 1 out: both
    layouts).  1 GiB of source, median of 3 blocks of 3 passes; bytes read +
    written over the time.  Each mix runs with plain and non-temporal loads
    and stores, grid-strided and in one contiguous range per workgroup; the
    best is the ceiling, and `hints` names it."""
    src = torch.empty(CEIL_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    d0 = torch.empty(CEIL_BYTES, dtype=torch.uint8, device="cuda")
    d1 = torch.empty(CEIL_BYTES // 2, dtype=torch.uint8, device="cuda")
    out, hints = {}, {}
    for name, mix in MIX_OF.items():
        moved = CEIL_BYTES + {probe.READ: 0, probe.COPY: CEIL_BYTES, probe.HALF: CEIL_BYTES // 2,
                              probe.SPLIT: CEIL_BYTES}[mix]
        for h in range(0, 8 * probe.NT_LOAD, probe.NT_LOAD):  # every subset of the three hint bits
            if mix == probe.READ and h & probe.NT_STORE:
                continue
            hn = "+".join(n for b, n in ((probe.NT_LOAD, "nt_load"), (probe.NT_STORE, "nt_store"),
                                         (probe.BLOCKED, "blocked")) if h & b) or "plain"
            ms = _time_ms(lambda: probe.stream(src, d0, d1 if mix == probe.SPLIT else None, mix | h), 3, ev)
            gbs = round(moved / (ms * 1e-3) / 1e9, 1)
            if gbs > out.get(name, 0.0):
                out[name], hints[name] = gbs, hn
    del src, d0, d1
    torch.cuda.empty_cache()
    return {"gbs": out, "hints": hints}


def _mfma_rate(ev: "HipEvents", varied: bool) -> dict:
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 60000
    clocks = torch.zeros(4 * cus, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    ms = _time_ms(lambda: probe.mfma(iters, cus, clocks, sink, varied), 1, ev)
    flops = cus * probe.MFMA_WAVES * iters * probe.MFMA_FLOPS_PER_ROUND
    c = clocks.view(-1, 4).cpu().numpy().astype(np.float64)
    wall_khz = probe.wall_clock_khz()
    ghz = float(np.median((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]))) * wall_khz / 1e6
    tf = flops / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "clock_ghz": round(ghz, 3), "cus": cus,
            "frac_of_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "peak_at_clock_tflops": round(PEAK_FP8_TFLOPS * ghz / PEAK_CLOCK_GHZ, 1)}


def mfma_ceiling(ev: "HipEvents") -> dict:
    """FP8 matrix-core rate this GPU sustains under full load (registers only,
    two waves per SIMD, one workgroup per compute unit), and the shader clock
    during it from the core and wall cycle counters of every workgroup: with
    fixed operands (top level: the clock limit) and with operands that change
    from product to product ("varied": the multipliers switch as in a GEMM
    over real data, which costs power and clock)."""
    out = _mfma_rate(ev, False)
    out["varied"] = _mfma_rate(ev, True)
    out["note"] = ("back-to-back 16x16x128 FP8 MFMAs from registers on every SIMD; clock = core cycles / wall "
                   "cycles x the wall counter's rate, median over workgroups; varied: four operand sets per "
                   "lane cycled so that each product multiplies other codes")
    return out


def calibrate_copy(nbytes: int):
    """A plain in-tree device copy of known size (fp8probe_stream COPY): what
    FETCH_SIZE / WRITE_SIZE read for it scales the counters taken on the
    path's kernels."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        probe.stream(src, dst, None, probe.COPY)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3, "kernel": "fp8probe_stream COPY"}))


# ---------------------------------------------------------------------------
# FP8-vs-BF16 GEMM speedup over K ("Mastering FP8 LLM training", Fig. 1)
# ---------------------------------------------------------------------------

SWEEP_K = (1024, 2048, 4096, 8192, 16384)


def _time_ms(fn, reps: int, ev: HipEvents) -> float:
    """Median over 3 blocks of `reps` back-to-back launches (fence-free events)."""
    fn()
    torch.cuda.synchronize()
    blocks = []
    for _ in range(3):
        ev.record(0, False)
        for _ in range(reps):
            fn()
        ev.record(0, True)
        torch.cuda.synchronize()
        blocks.append(ev.ms(0) / reps)
    return float(np.median(blocks))


def speedup_sweep(M: int, N: int, ks, reps: int):
    """One JSON line per K: TFLOP/s of the BF16 GEMM (same kernel, BF16
    matrix-core instruction) and of the scaled FP8 GEMM in each scaling
    recipe, and each recipe's speedup over BF16.  Operands: N(0, 1) BF16
    A [M x K], N(0, 0.02) B [N x K], quantized by the library with the
    recipe's own granularity (rows of A 1x128 / 1x32, B per recipe).
    hipBLASLt's BF16 GEMM (torch.matmul) is timed beside it for context."""
    ev = HipEvents(1)
    recipes = (("tensor", fm.TENSOR_CURRENT, fm.TENSOR_CURRENT, fm.GEMM_TENSOR),
               ("channel", fm.CHANNEL, fm.CHANNEL, fm.GEMM_CHANNEL),
               ("128x128_128x128", fm.BLOCK_128x128, fm.BLOCK_128x128, fm.GEMM_BLOCK_128x128_128x128),
               ("1x128_128x128", fm.BLOCK_1x128, fm.BLOCK_128x128, fm.GEMM_BLOCK_1x128_128x128),
               ("1x128_1x128", fm.BLOCK_1x128, fm.BLOCK_1x128, fm.GEMM_BLOCK_1x128_1x128),
               ("mx_1x32", fm.MX_1x32, fm.MX_1x32, fm.GEMM_MX_1x32))
    for K in ks:
        g = torch.Generator(device="cuda")
        g.manual_seed(4242 + K)
        a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        b = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        flop = 2.0 * M * N * K
        c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        line = {"sweep": "fp8_vs_bf16_gemm", "M": M, "N": N, "K": K, "out": "bf16"}
        t_bf = _time_ms(lambda: fm.bf16_gemm(a, b, c=c), reps, ev)
        line["bf16"] = {"ms": round(t_bf, 4), "tflops": round(flop / t_bf / 1e9, 1)}
        bt = b.t().contiguous()  # [K x N]; a plain 2-D product, no transposed view
        t_lt = _time_ms(lambda: torch.mm(a, bt, out=c), reps, ev)
        line["bf16_hipblaslt"] = {"ms": round(t_lt, 4), "tflops": round(flop / t_lt / 1e9, 1)}
        for name, ra, rb, rg in recipes:
            qa = fm.quantize(a, ra, fm.E4M3, fm.ROW)
            qb = fm.quantize(b, rb, fm.E4M3, fm.ROW)
            sa = qa.scale_inv if rg == fm.GEMM_TENSOR else qa.s_row
            sb = qb.scale_inv if rg == fm.GEMM_TENSOR else qb.s_row
            t = _time_ms(lambda: fm.gemm(qa.q_row, fm.E4M3, sa, qb.q_row, fm.E4M3, sb, rg, K,
                                         M=M, N=N, c=c), reps, ev)
            line[name] = {"ms": round(t, 4), "tflops": round(flop / t / 1e9, 1),
                          "speedup_vs_bf16": round(t_bf / t, 3)}
            del qa, qb
        print(json.dumps(line), flush=True)
        del a, b, c
        torch.cuda.empty_cache()


def latency_line(cfg: workloads.Config, args, ev: "HipEvents") -> dict:
    """Microseconds per step of the tiny blockwise case: quantize A (1x128),
    quantize B (128x128), fprop GEMM -- launched eagerly, and as one HIP
    graph replayed (the captured launches are the same three)."""
    x, w = workloads.make(cfg.X, "cuda"), workloads.make(cfg.W, "cuda")
    M, N, K = cfg.M, cfg.N, cfg.K
    c = lambda a, b: (a + b - 1) // b  # noqa: E731
    qx = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, c(K, 128), dtype=torch.float32, device="cuda")
    qw = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(c(N, 128), c(K, 128), dtype=torch.float32, device="cuda")
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ops = [
        ("quant_a_1x128", lambda: _ok(fm.fp8_quantize(x, fm.IN_BF16, M, K, K, fm.BLOCK_1x128, fm.E4M3, fm.ROW, 0,
                                                      qx, K, sx, None, 0, None, None, None, None, None))),
        ("quant_b_128x128", lambda: _ok(fm.fp8_quantize(w, fm.IN_BF16, N, K, K, fm.BLOCK_128x128, fm.E4M3, fm.ROW,
                                                        0, qw, K, sw, None, 0, None, None, None, None, None))),
        ("gemm_fprop", lambda: _ok(fm.fp8_gemm_scaled(qx, fm.E4M3, sx, K, qw, fm.E4M3, sw, K,
                                                      fm.GEMM_BLOCK_1x128_128x128, fm.LAYOUT_TN, M, N, K, y,
                                                      fm.OUT_BF16, N))),
    ]

    def step():
        for _, f in ops:
            f()

    reps = 200
    for _ in range(args.warmup):
        step()
    eager = _time_ms(step, reps, ev) * 1e3
    per_op = {name: round(_time_ms(f, reps, ev) * 1e3, 2) for name, f in ops}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()  # warm the capture stream
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    replay = _time_ms(graph.replay, reps, ev) * 1e3
    # the floor: three launches of an empty kernel, eagerly and as a graph
    empty3 = lambda: [probe.empty(1, 256) for _ in range(3)]  # noqa: E731
    floor_eager = _time_ms(empty3, reps, ev) * 1e3
    floor_graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        empty3()
        with torch.cuda.graph(floor_graph, stream=side):
            empty3()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    floor_replay = _time_ms(floor_graph.replay, reps, ev) * 1e3
    return {
        "metric": "FP8 blockwise step latency (quantize A 1x128, quantize B 128x128, fprop GEMM)",
        "value": round(replay, 2), "unit": "us", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": cfg.name, "recipe": cfg.recipe, "M": M, "N": N, "K": K, "inputs": "bf16",
                   "outputs": "bf16"},
        "eager_us": round(eager, 2), "graph_replay_us": round(replay, 2), "kernels_us": per_op,
        "launch_floor_us": {"eager": round(floor_eager, 2), "graph_replay": round(floor_replay, 2),
                            "what": "three launches of an empty kernel (fp8probe_empty, one workgroup)"},
        "note": "latency-bound case: value is one replay of a HIP graph holding the three launches; eager_us the "
                "same three launches issued from Python; median of 3 blocks of 200 back-to-back steps",
    }


def _roofline(name: str, flops: int, launch_ms, ceiling: dict, workload: str) -> dict:
    ms = float(np.mean(launch_ms))
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": name, "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "frac_of_mfma_ceiling": round(achieved / ceiling["tflops"], 4),
            "frac_at_probe_clock": round(achieved / ceiling["peak_at_clock_tflops"], 4),
            "frac_of_mfma_ceiling_varied": round(achieved / ceiling["varied"]["tflops"], 4),
            "traffic": _traffic(workload, name), "launches_timed": len(launch_ms),
            "launch_ms_mean": round(ms, 4), "flops_per_launch": flops}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(workloads.CONFIGS))
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies the steps rotate over (0: at least 4, and enough that every "
                         "input's copies exceed 512 MiB, twice the Infinity Cache)")
    ap.add_argument("--event-every", type=int, default=2, metavar="E",
                    help="bracket the dominant and fprop GEMMs with timing events in every E-th timed step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the HBM and matrix-core ceiling probes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain in-tree device copy of BYTES (reference for the HBM byte counters)")
    ap.add_argument("--speedup-sweep", action="store_true",
                    help="only print the FP8-vs-BF16 GEMM speedup over K (one JSON line per K)")
    ap.add_argument("--sweep-mn", type=int, default=8192, help="M = N of the speedup sweep")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the quantize + GEMM path runs on one GPU's share; the sharded design is described, not run)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fm.load()
    if args.speedup_sweep:
        speedup_sweep(args.sweep_mn, args.sweep_mn, SWEEP_K, 10)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    cfg = workloads.CONFIGS[args.workload]
    ev = HipEvents(1)
    if cfg.G is None:
        print(json.dumps(latency_line(cfg, args, ev)))
        return

    if args.rotate <= 0:
        smallest = min(t.rows * t.cols * 2 for t in (cfg.X, cfg.W, cfg.G))  # BF16 bytes
        args.rotate = max(4, -(-(512 << 20) // smallest) + 1)
    step = Step(cfg, args.rotate)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step.run(i)
    torch.cuda.synchronize()

    # per-op breakdown: each op alone, `reps` back-to-back launches over the
    # rotating input copies between one pair of events
    reps = 10
    op_ms = []
    for _, _, _, fn in step.ops:
        fn(0)
        torch.cuda.synchronize()
        ev.record(0, False)
        for r in range(reps):
            fn(r % step.rotate)
        ev.record(0, True)
        torch.cuda.synchronize()
        op_ms.append(ev.ms(0) / reps)

    # dominant kernel: the GEMM with the largest share of the step; fprop beside it
    gemm_i = [i for i, op in enumerate(step.ops) if op[1] == "gemm"]
    dom_i = max(gemm_i, key=lambda i: op_ms[i])
    fprop_i = next(i for i in gemm_i if step.ops[i][0] == "gemm_fprop")
    bracket = sorted({dom_i, fprop_i})

    # the timed region: K whole steps; the bracketed GEMMs carry (fence-free)
    # events in every E-th step
    for i in range(2):
        step.run(args.warmup + i)
    sampled = [i for i in range(args.steps) if i % args.event_every == 0]
    tev = {i: HipEvents(len(sampled)) for i in bracket}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % args.event_every == 0:
            j = i // args.event_every
            for k, (_, _, _, fn) in enumerate(step.ops):
                if k in tev:
                    tev[k].record(j, False)
                fn((args.warmup + i) % step.rotate)
                if k in tev:
                    tev[k].record(j, True)
        else:
            step.run(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = {k: [tev[k].ms(j) for j in range(len(sampled))] for k in bracket}

    # what an empty event pair costs the queue (the bracket's own overhead)
    empty = []
    for _ in range(5):
        ev.record(0, False)
        ev.record(0, True)
        torch.cuda.synchronize()
        empty.append(ev.ms(0) * 1e3)

    ceil_hbm = hbm_ceilings(ev) if not args.no_probes else None
    nan = float("nan")
    ceil_mfma = mfma_ceiling(ev) if not args.no_probes else {"tflops": nan, "peak_at_clock_tflops": nan,
                                                             "varied": {"tflops": nan}}

    kernels = {}
    for (name, kind, work, _), ms in zip(step.ops, op_ms):
        ent = {"ms": round(ms, 4)}
        if kind == "gemm":
            tf = work / (ms * 1e-3) / 1e12
            ent.update({"tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)})
        elif kind == "quant":
            gbs = work / (ms * 1e-3) / 1e9
            ent.update({"gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": work})
            mix = "ROW_AND_COL" if "row_col" in name else "ROW"
            if ceil_hbm:
                ent.update({"ceiling_mix": mix, "frac_hbm_ceiling": round(gbs / ceil_hbm["gbs"][mix], 4)})
        kernels[name] = ent

    value = step.gemm_flops() / (ms_step * 1e-3) / 1e12
    dom, fp = step.ops[dom_i], step.ops[fprop_i]
    out = {
        "metric": "FP8 scaled GEMM TFLOPS (fprop/dgrad/wgrad) + quantize GB/s, % of MI355X peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": args.workload, "recipe": cfg.recipe, "M": cfg.M, "N": cfg.N, "K": cfg.K,
                   "gemms": list(cfg.gemms), "inputs": "bf16", "outputs": "bf16",
                   "rotating_input_copies": args.rotate},
        "roofline": _roofline(dom[0], dom[2], launch_ms[dom_i], ceil_mfma, args.workload),
        "roofline_fprop": _roofline(fp[0], fp[2], launch_ms[fprop_i], ceil_mfma, args.workload),
        "event_pair_empty_us": round(float(np.median(empty)), 2),
        "kernels": kernels,
        "mfma_ceiling": ceil_mfma if not args.no_probes else None,
        "hbm_ceiling": ({"gbs": ceil_hbm["gbs"], "hints": ceil_hbm["hints"], "source_bytes": CEIL_BYTES,
                         "note": "in-tree streams (libfp8mi_probe.so), best of plain / non-temporal loads and "
                                 "stores, strided / blocked: bytes read + written / time; ROW = 2 bytes in, 1 out; ROW_AND_COL = 2 "
                                 "in, 1 + 1 out"} if ceil_hbm else None),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
