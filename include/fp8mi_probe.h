/*
 * fp8mi_probe.h -- C ABI of libfp8mi_probe.so: measurement kernels that tell
 * what this GPU sustains, so that the FP8 path's kernels can be judged
 * against the chip rather than against a datasheet alone.  Not part of the
 * method; nothing in libfp8mi.so calls them.
 *
 * Why: "From FP16 to FP8", sec. 3.1 judges an FP8 GEMM benchmark by the
 * fraction of the theoretical rate it reaches.  The datasheet peaks assume
 * the top clock and ideal memory; these kernels measure the matrix-core
 * rate and shader clock under full FP8 MFMA load (with fixed and with
 * varied operands), and the HBM rate of plain
 * streams with the quantize kernels' read:write byte mixes, and the cost
 * of an empty launch.
 *
 * Conventions as in fp8mi.h: device pointers, `stream` a hipStream_t, int
 * status (FP8MI_OK = 0 or a negative FP8MI_ERR_* code), nothing allocated.
 */
#ifndef FP8MI_PROBE_H
#define FP8MI_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* read:write mixes of fp8probe_stream */
#define FP8PROBE_READ 0  /* read n16 chunks, write nothing                       */
#define FP8PROBE_COPY 1  /* dst0[i] = src[i], i < n16                            */
#define FP8PROBE_HALF 2  /* dst0[i] = src[2i] ^ src[2i+1]: 2 bytes in, 1 out      */
                         /* (a BF16 -> FP8 cast writing one code layout)          */
#define FP8PROBE_SPLIT 3 /* dst0[i] = src[2i], dst1[i] = src[2i+1]: 2 in, 1+1 out */
                         /* (a cast writing both code layouts)                   */
/* access hints, OR-ed into `mix` */
#define FP8PROBE_NT_LOAD 16  /* non-temporal loads (the data is read once)    */
#define FP8PROBE_NT_STORE 32 /* non-temporal stores                           */
#define FP8PROBE_BLOCKED 64  /* each workgroup streams one contiguous range  */
                             /* (default: grid-strided)                       */

/* fp8probe_stream -- one streaming pass over n16 16-byte chunks of src
 * (16-byte aligned) by eight workgroups per compute unit, eight 16-byte
 * loads in flight per thread, grid-strided or (FP8PROBE_BLOCKED) in one
 * contiguous range per workgroup.  dst0 (and dst1 for SPLIT) receive n16 (COPY) or
 * n16 / 2 (HALF, SPLIT) chunks; READ stores at most one 16-byte chunk into
 * dst0 (only when the XOR of the data is a fixed sentinel, which keeps the
 * reads live), so dst0 must hold 16 bytes.  HALF and SPLIT need n16 even.
 * Returns FP8MI_OK, -1 (NULL pointer), -2 (bad mix), -3 (n16 < 0 or odd
 * where it must be even), -5 (misaligned) or -6 (launch failed).  `mix` is
 * one of the mixes above, optionally OR-ed with any of FP8PROBE_NT_LOAD,
 * FP8PROBE_NT_STORE and FP8PROBE_BLOCKED. */
int fp8probe_stream(const void* src, int64_t n16, void* dst0, void* dst1, int mix, void* stream);

/* fp8probe_mfma -- `iters` rounds of eight independent 16x16x128 FP8
 * matrix-core products (v_mfma_f32_16x16x128_f8f6f4, E4M3 operands held in
 * registers, no memory traffic) on every SIMD: two waves per SIMD, one
 * workgroup of eight waves per compute unit (each holds 96 KB of LDS, so no
 * second one fits), `workgroups` of them.  Flops
 * = workgroups * 8 waves * iters * 8 * 65536.  clocks [4 * workgroups]
 * receives per workgroup the core cycle counter and the constant-rate wall
 * counter at the start and the end of its loop (c0, c1, w0, w1), so the
 * shader clock under this load is (c1 - c0) / (w1 - w0) times the wall
 * counter's rate (hipDeviceAttributeWallClockRate).  sink: one float, never
 * written in practice (keeps the products live).
 * Returns FP8MI_OK, -1 (NULL pointer), -3 (iters or workgroups < 1) or -6. */
int fp8probe_mfma(int iters, int workgroups, uint64_t* clocks, float* sink, void* stream);

/* fp8probe_mfma_varied -- fp8probe_mfma with operands that change from one
 * product to the next: each lane holds four sets of E4M3 codes drawn from
 * a hash of its position (the lowest exponent bit cleared, so no code is
 * NaN) and the eight products of a round cycle through them, so that the
 * multipliers switch as they do in a GEMM over real data.  Switching costs
 * power, so this load runs at a lower clock than fp8probe_mfma's fixed
 * operands: its rate is the matrix-core ceiling a GEMM over real data can
 * approach, fp8probe_mfma's the chip's clock limit.  Same arguments, flops,
 * clocks layout and return values as fp8probe_mfma. */
int fp8probe_mfma_varied(int iters, int workgroups, uint64_t* clocks, float* sink, void* stream);

/* fp8probe_empty -- one launch of a kernel with an empty body, `workgroups`
 * workgroups of `threads` threads: the cost of a dispatch alone, the floor
 * under a launch-latency-bound step.  Returns FP8MI_OK, -3 (workgroups < 1,
 * threads outside 1..1024) or -6. */
int fp8probe_empty(int workgroups, int threads, void* stream);

/* fp8probe_wall_clock_khz -- rate of the constant wall counter that
 * fp8probe_mfma records, in kHz, for the device `stream` runs on (NULL: the
 * current device).  Returns the rate (> 0) or -6 if the query failed. */
int fp8probe_wall_clock_khz(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8MI_PROBE_H */
