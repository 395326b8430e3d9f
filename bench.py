"""Benchmark of the FP8 training hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the whole path over one batch of synthetic inputs:
quantize every GEMM operand with the workload's recipe (including the
transposed layouts the backward GEMMs read), the delayed-scaling history
update where the recipe has one, then the fprop / dgrad (/ wgrad) scaled FP8
GEMMs.  Inputs are resident in HBM before timing starts; R rotating copies of
every input (default 4, > 256 MB in total) keep each step's reads from being
served by the previous step's Infinity Cache contents.

Prints ONE JSON line.  `value` is GEMM FLOP of the step / step time (TFLOP/s),
so quantization time counts against it.  Per-kernel figures (TFLOP/s or GB/s
against the MI355X peaks) are under "kernels", each op timed on its own over
back-to-back launches; "roofline" is the dominant kernel's, timed inside the
timed steps with HIP events on the stream it runs on, in every 4th step
(--event-every).  The events are created without the system-scope release
fence (a fenced event writes back and invalidates the caches and stalls the
queue for several microseconds); even so each record costs the queue about
4.5 us, which is why not every step carries them.  "hbm_copy" is a 1 GiB
device copy timed on the same GPU: each cast's "frac_copy" holds its GB/s
against that achievable rate, "frac_hbm_peak" against the 8 TB/s
specification.  "cpu_baseline" is the CPU oracle timed on a
bounded sample of the same step and extrapolated to the full step (rank 0,
one thread).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_scaled_quantization_scale_amd as fm  # noqa: E402
import workloads  # noqa: E402

PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, GB/s
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 / MXFP8 matrix peak, TFLOP/s
DEFAULT_WORKLOAD = "llama3_8b_attn_tensor"


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
                                   fm.GEMM_TENSOR, M, N, K, self.y, fm.OUT_BF16, N))

        def dgrad(r):
            # dX[M x K] = dY[M x N] . W[N x K]: A = dY codes, B = W^T codes [K x N]
            _ok(fm.fp8_gemm_scaled(self.qg, fm.E5M2, st.scale_inv, N, self.qwt, fm.E4M3, self.siw, N,
                                   fm.GEMM_TENSOR, M, K, N, self.dx, fm.OUT_BF16, K))

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
                                   fm.GEMM_BLOCK_1x128_128x128, M, N, K, self.y, fm.OUT_BF16, N))

        def dgrad(r):
            _ok(fm.fp8_gemm_scaled(self.qg, fm.E4M3, self.sg, N, self.qwt, fm.E4M3, self.swt, N,
                                   fm.GEMM_BLOCK_1x128_128x128, M, K, N, self.dx, fm.OUT_BF16, K))

        def wgrad(r):
            # dW[N x K] = dY^T[N x M] . X[M x K]: both operands blocked along M
            _ok(fm.fp8_gemm_scaled(self.qgt, fm.E4M3, self.sgt, M, self.qxt, fm.E4M3, self.sxt, M,
                                   fm.GEMM_BLOCK_1x128_1x128, N, K, M, self.dw, fm.OUT_BF16, K))

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
                                   fm.GEMM_MX_1x32, M, N, K, self.y, fm.OUT_BF16, N))

        def dgrad(r):
            _ok(fm.fp8_gemm_scaled(self.qg, fm.E4M3, self.sg, N, self.qwt, fm.E4M3, self.swt, N,
                                   fm.GEMM_MX_1x32, M, K, N, self.dx, fm.OUT_BF16, K))

        def wgrad(r):
            _ok(fm.fp8_gemm_scaled(self.qgt, fm.E4M3, self.sgt, M, self.qxt, fm.E4M3, self.sxt, M,
                                   fm.GEMM_MX_1x32, N, K, M, self.dw, fm.OUT_BF16, K))

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

def cpu_baseline(cfg: workloads.Config, rows: int = 1024, wrows: int = 1024):
    """Time the oracle on a bounded sample of the step -- `rows` token rows of
    X and G, `wrows` rows of W, and the GEMM outputs of those rows -- and
    extrapolate to the full step: token-row costs x M/rows, weight-row costs
    x N/wrows, GEMM cost x (M/rows)(N/wrows) per GEMM (dgrad and wgrad do the
    same contraction work as fprop)."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle

    M, N, K = cfg.M, cfg.N, cfg.K
    x = workloads.make(cfg.X, rows=rows).float().numpy()
    w = workloads.make(cfg.W, rows=wrows).float().numpy()
    g = workloads.make(cfg.G, rows=rows).float().numpy()
    n_gemms = len(cfg.gemms)

    def run():
        """One pass of the oracle over the sample: (t0, t1, t2, t3)."""
        if cfg.recipe == "tensor":
            t0 = time.perf_counter()
            qx, _, six, _, _ = oracle.quantize_current("e4m3", x)
            h = oracle.History("e5m2", 200)
            qg, am = oracle.quantize_delayed("e5m2", g, h.scale)
            h.update(am)
            t1 = time.perf_counter()
            qw, _, siw, _, _ = oracle.quantize_current("e4m3", w)
            np.ascontiguousarray(qw.T)
            t2 = time.perf_counter()
            oracle.gemm_ref(oracle.dequant("e4m3", qx, six), oracle.dequant("e4m3", qw, siw))
            t3 = time.perf_counter()
            return t0, t1, t2, t3
        if cfg.recipe == "block":
            quant = lambda v, br, bc: oracle.quantize_blocks("e4m3", v, br, bc)  # noqa: E731
            deq = oracle.dequant
            rb, cb, wb, wcb = (1, 128), (128, 1), (128, 128), None
        else:
            quant = lambda v, br, bc: oracle.quantize_mx("e4m3", v, br, bc)  # noqa: E731
            deq = oracle.dequant_mx
            rb, cb, wb, wcb = (1, 32), (32, 1), (1, 32), (32, 1)
        t0 = time.perf_counter()
        qx, gx, _ = quant(x, *rb)
        quant(x, *cb)
        quant(g, *rb)
        quant(g, *cb)
        t1 = time.perf_counter()
        qw, gw, _ = quant(w, *wb)
        if wcb is not None:
            quant(w, *wcb)
        t2 = time.perf_counter()
        oracle.gemm_ref(deq("e4m3", qx, gx, *rb), deq("e4m3", qw, gw, *wb))
        t3 = time.perf_counter()
        return t0, t1, t2, t3

    def extrapolate(t):
        t0, t1, t2, t3 = t
        return ((t1 - t0) * (M / rows) + (t2 - t1) * (N / wrows)
                + (t3 - t2) * (M / rows) * (N / wrows) * n_gemms)

    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx is not None:
        ctx.__enter__()
    try:
        t0, t1, t2, t3 = run()
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    # the same sample with the float64 GEMM on every BLAS thread (the C
    # quantizer is single-threaded either way)
    ta = run()
    blas_threads = 0
    if threadpool_limits is not None:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"],
                           default=0)
    full = extrapolate((t0, t1, t2, t3))
    flops = n_gemms * 2.0 * M * N * K
    return {
        "value": round(flops / full / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"oracle on {rows} of {M} token rows of X and G, {wrows} of {N} weight rows, and "
                   f"the {rows}x{wrows} GEMM outputs they give (float64 numpy, 1 thread); measured "
                   f"{(t3 - t0):.2f} s, extrapolated to the full step ({full:.1f} s)"),
        "all_cores": {"value": round(flops / extrapolate(ta) / 1e12, 6), "blas_threads": blas_threads,
                      "note": "same sample, float64 GEMM on every BLAS thread; the C quantizer stays on one"},
        "host_cpu": _cpu_model(),
        "host_cpus_visible": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count(),
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
    """Hash of the sources that define the kernels and their launch
    configuration (the HIP files and the two internal headers; the C ABI's
    host-side validation in api.cpp does not change what a kernel moves)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_scaled_quantization_scale_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith(".hip") or f in ("device.hpp", "launch.hpp"):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
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


COPY_BYTES = 1 << 30


def measure_copy_gbs(ev: "HipEvents") -> float:
    """What this GPU sustains for a plain device copy (1 GiB, MALL-cold):
    bytes read + bytes written over the median time of 3 blocks of 3 copies
    -- the ceiling the bandwidth-bound casts are held against beside the 8 TB/s
    spec figure."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = _time_ms(lambda: dst.copy_(src), 3, ev)
    del src, dst
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def calibrate_copy(nbytes: int):
    """A plain device-to-device copy of known size: what FETCH_SIZE / WRITE_SIZE
    read for it scales the counters taken on the path's kernels."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}))


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(workloads.CONFIGS))
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--event-every", type=int, default=4, metavar="E",
                    help="bracket the dominant kernel with timing events in every E-th timed step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (reference for the HBM byte counters)")
    ap.add_argument("--speedup-sweep", action="store_true",
                    help="only print the FP8-vs-BF16 GEMM speedup over K (one JSON line per K)")
    ap.add_argument("--sweep-mn", type=int, default=8192, help="M = N of the speedup sweep")
    args = ap.parse_args()
    if args.speedup_sweep:
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(2)
        speedup_sweep(args.sweep_mn, args.sweep_mn, SWEEP_K, 10)
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the quantize + GEMM path runs on one GPU's share)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fm.load()
    cfg = workloads.CONFIGS[args.workload]
    if cfg.G is None:
        print(f"workload {args.workload} is a parity case, not a bench line", file=sys.stderr)
        sys.exit(2)

    step = Step(cfg, args.rotate)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step.run(i)
    torch.cuda.synchronize()

    # per-op breakdown: each op alone, `reps` back-to-back launches over the
    # rotating input copies between one pair of events
    reps = 10
    ev = HipEvents(1)
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
    copy_gbs = measure_copy_gbs(ev)
    kernels = {}
    for (name, kind, work, _), ms in zip(step.ops, op_ms):
        ent = {"ms": round(ms, 4)}
        if kind == "gemm":
            tf = work / (ms * 1e-3) / 1e12
            ent.update({"tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)})
        elif kind == "quant":
            gbs = work / (ms * 1e-3) / 1e9
            ent.update({"gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                        "frac_copy": round(gbs / copy_gbs, 4), "algorithmic_bytes": work})
        kernels[name] = ent

    # dominant kernel: the GEMM with the largest share of the step
    dom_i = max((i for i, op in enumerate(step.ops) if op[1] == "gemm"), key=lambda i: op_ms[i])
    dom = step.ops[dom_i]

    # the timed region: K whole steps; the dominant kernel is bracketed by
    # (fence-free) events in every EVERY-th step.  Each event record still
    # costs the queue about 4.5 us (visible as gaps in a kernel trace), so
    # bracketing every step would charge ~9 us of instrumentation to each.
    for i in range(2):
        step.run(args.warmup + i)
    sampled = [i for i in range(args.steps) if i % args.event_every == 0]
    tev = HipEvents(len(sampled))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % args.event_every == 0:
            step.run(args.warmup + i, dom_i, tev, i // args.event_every)
        else:
            step.run(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    dom_launch_ms = [tev.ms(j) for j in range(len(sampled))]

    dom_ms = float(np.mean(dom_launch_ms))
    achieved = dom[2] / (dom_ms * 1e-3) / 1e12
    traffic = _traffic(args.workload, dom[0])
    value = step.gemm_flops() / (ms_step * 1e-3) / 1e12
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
        "roofline": {"bound": "mfma", "kernel": dom[0], "achieved": round(achieved, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                     "launches_timed": len(dom_launch_ms)},
        "kernels": kernels,
        "hbm_copy": {"gbs": round(copy_gbs, 1), "bytes": COPY_BYTES,
                     "note": "device-to-device copy on this GPU, read + write bytes / time; frac_copy of a cast is "
                             "its algorithmic GB/s over this"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
