/*
 * fp8mi.h -- C ABI of the MI355X (gfx950) FP8 scaled-quantization and
 * scaled-FP8-GEMM library (libfp8mi.so).
 *
 * What is computed (cited by page and section; the pages are web articles
 * on FP8 training):
 *   [P1] "2025 technical guide: FP8 quantized training" (blog.gitcode.com)
 *        sec. 1.1  E4M3 / E5M2 bit layouts;
 *        sec. 2.1  per-tensor scaling: delayed (amax history over the past
 *                  steps, usually 200, scale from the history maximum) and
 *                  current (amax of the tensor being cast);
 *        sec. 2.2  blockwise scaling: 1x128 tiles for inputs and gradients,
 *                  128x128 tiles for weights, one scale per tile;
 *        sec. 2.3  MXFP8: 1x32 blocks with E8M0 power-of-two scales;
 *        sec. 3.1  the three GEMMs (fprop, dgrad, wgrad) take quantized
 *                  inputs and keep BF16/FP32 outputs.
 *   [P2] "From FP16 to FP8" (bjdmk.com.cn/news/5220490) sec. 1-2: E5M2
 *        range 57344 .. 6.1e-5, bias 15; sec. 3.3: DelayedScaling with
 *        margin and an update every step.
 *   [P3] "Mastering FP8 LLM training" (nmedialink.com) strategies 1-4
 *        (delayed, current, sub-channel blocks that need re-quantization
 *        on transpose, MXFP8) and Fig. 1 (GEMM cost by scaling granularity).
 *   [P4] "FP8 training support" (bjdmk.com.cn/news/366077) "Why FP8?":
 *        E4M3 for weights/activations, E5M2 for gradients; a per-tensor
 *        scale maps the FP32 range onto the FP8 range.
 *
 * Numerics (identical bit for bit to the CPU oracle):
 *   E4M3 = OCP E4M3FN (max 448, subnormals, NaN 0x7F/0xFF, no Inf);
 *   E5M2 = OCP E5M2 (max 57344, subnormals, Inf 0x7C/0xFC).
 *   code = enc(fl32(x * s)): one binary32 multiply, then round to nearest,
 *   ties to the even code, saturating (|v| >= max and +-Inf give +-max),
 *   NaN gives 0x7F, -0 gives 0x80.
 *   s = fl32(max / amax) * 2^-margin (amax == 0 or non-finite: s = 1;
 *   +Inf: FLT_MAX); s_inv = fl32(1 / s) is the dequantisation scale the
 *   GEMM consumes.  MX: E8M0 byte e + 127 with e = ceil(log2(amax / max))
 *   clamped to [-127, 127] (amax == 0: 127; non-finite: 0xFF), elements
 *   enc(fl32(x * 2^-e)).
 *
 * Conventions:
 *   - Every matrix is row-major with an explicit leading dimension counted
 *     in elements.  Tensor and scale pointers are DEVICE pointers; `stream`
 *     is a hipStream_t (NULL = the null stream).
 *   - The library allocates nothing, keeps no state between calls and
 *     never synchronises the host: all work is enqueued on `stream`.
 *     Calls that write the same buffers on different streams race.
 *   - Return values report host-checkable errors only.  Data-dependent
 *     conditions (NaN/Inf inputs) are reported through device outputs:
 *     a non-finite amax, and the `nonfinite` counters.
 *   - Weights are stored [out x in] = [N x K], so every GEMM operand is
 *     row-major with the contraction index contiguous ("TN" layout).
 */
#ifndef FP8MI_H
#define FP8MI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define FP8MI_OK 0
#define FP8MI_ERR_NULL (-1)        /* a required pointer is NULL            */
#define FP8MI_ERR_ENUM (-2)        /* unknown recipe / format / dtype value */
#define FP8MI_ERR_SHAPE (-3)       /* negative size, ld too small, margin   */
#define FP8MI_ERR_UNSUPPORTED (-4) /* valid values, combination not built   */
#define FP8MI_ERR_ALIGN (-5)       /* pointer or ld breaks its alignment     */
#define FP8MI_ERR_HIP (-6)         /* a HIP launch failed                   */

/* ---- enums ------------------------------------------------------------ */
#define FP8MI_E4M3 0 /* OCP E4M3FN */
#define FP8MI_E5M2 1 /* OCP E5M2   */

#define FP8MI_IN_BF16 0
#define FP8MI_IN_FP32 1

#define FP8MI_OUT_BF16 0
#define FP8MI_OUT_FP32 1

/* quantize recipes [P1 sec. 2.1-2.3] */
#define FP8MI_TENSOR_CURRENT 0 /* amax of x now -> s; writes amax[0], scale, scale_inv */
                               /* (amax: float[FP8MI_AMAX_SLOTS], the rest scratch)     */
#define FP8MI_TENSOR_DELAYED 1 /* cast with *scale; max-accumulates max|x| into the     */
                               /* amax accumulator float[FP8MI_AMAX_SLOTS]             */
#define FP8MI_BLOCK_1x128 2    /* ROW: 1x128 along cols; COL: 128x1 down rows            */
#define FP8MI_BLOCK_128x128 3  /* one scale per 128x128 tile                             */
#define FP8MI_MX_1x32 4        /* ROW: 1x32 along cols; COL: 32x1 down rows; E8M0 bytes  */
#define FP8MI_CHANNEL 5        /* ROW: one scale per row; COL: one per column [P3 Fig. 1] */
#define FP8MI_MX_1x32_OCP 6    /* MX_1x32 with the OCP floor rule for the E8M0 exponent */

/* which code layouts to write */
#define FP8MI_ROW 1         /* q_row [rows x cols]                          */
#define FP8MI_COL 2         /* q_col [cols x rows] = codes written transposed */
#define FP8MI_ROW_AND_COL 3 /* both, from one read of x                      */

/* GEMM scale recipes [P1 sec. 2.1-2.3, 3.1] */
#define FP8MI_GEMM_TENSOR 0            /* s_a, s_b: one float each (scale_inv)              */
#define FP8MI_GEMM_BLOCK_1x128_128x128 1 /* s_a [M x ceil(K/128)], s_b [ceil(N/128) x ceil(K/128)] */
#define FP8MI_GEMM_BLOCK_1x128_1x128 2   /* s_a [M x ceil(K/128)], s_b [N x ceil(K/128)]      */
#define FP8MI_GEMM_MX_1x32 3             /* s_a [M x ceil(K/32)], s_b [N x ceil(K/32)] E8M0   */
#define FP8MI_GEMM_BLOCK_128x128_128x128 4 /* s_a [ceil(M/128) x ceil(K/128)], s_b [ceil(N/128) x ceil(K/128)] */
#define FP8MI_GEMM_CHANNEL 5             /* s_a [M], s_b [N]: one float per row of A and of B  */

/* GEMM operand layouts [P1 sec. 3.1: fprop, dgrad and wgrad read the same
 * tensors in different orientations; P3 strategy 3: a block-scaled operand
 * used transposed is re-quantized, so every GEMM can read codes whose
 * contraction index is contiguous].  fp8_quantize writes both orientations
 * (ROW_AND_COL), hence one layout serves all three GEMMs. */
#define FP8MI_LAYOUT_TN 0 /* a [M x K] and b [N x K], row-major, K contiguous in both */

/* Floats in the amax array of a per-tensor cast.  Each workgroup of a
 * TENSOR_DELAYED cast max-accumulates into a slot of its own with plain
 * loads and stores, and fp8_amax_history_update folds the slots into the
 * step's amax; a TENSOR_CURRENT cast keeps its per-workgroup partial maxima
 * in slots 1.. and the result in slot 0.  (Atomics on one address serialise
 * on MI355X; with a thousand workgroups they would cost as much as the cast
 * itself.) */
#define FP8MI_AMAX_SLOTS 1024

/* ---- entry points ----------------------------------------------------- */

/* fp8_quantize -- scaled cast of x [rows x cols] (BF16 or FP32) to FP8 codes.
 * [P1 sec. 2.1 (per-tensor current / delayed), 2.2 (1x128, 128x128),
 *  2.3 (MX 1x32 + E8M0); P3 strategy 3 (re-quantize for the transposed use)]
 *
 *   x, x_dtype, rows, cols, ld_x : input, ld_x >= cols elements.
 *   recipe, fmt, orient, margin  : FP8MI_* values above; margin in [0, 64]
 *                                  (per-tensor and FP32-scale block recipes;
 *                                  ignored by MX).
 *   q_row, ld_q_row, s_row       : ROW output.  Codes [rows x cols].
 *        BLOCK_1x128   s_row = float [rows x ceil(cols/128)]   (s_inv per block)
 *        BLOCK_128x128 s_row = float [ceil(rows/128) x ceil(cols/128)]
 *        MX_1x32       s_row = uint8 [rows x ceil(cols/32)]    (E8M0 bytes)
 *        MX_1x32_OCP   as MX_1x32; the exponent is floor(log2(amax)) - emax
 *                      (emax 8 for E4M3, 15 for E5M2) as the OCP microscaling
 *                      specification computes it, so elements above max
 *                      saturate; MX_1x32 takes the smallest power of two
 *                      under which none does.
 *        CHANNEL       s_row = float [rows]  (s_inv of each whole row)
 *        TENSOR_*      s_row unused.
 *   q_col, ld_q_col, s_col       : COL output.  Codes of x^T, [cols x rows].
 *        BLOCK_1x128   blocks run 128 rows down each column:
 *                      s_col = float [cols x ceil(rows/128)]
 *        BLOCK_128x128 same tiles and scales as ROW, grid transposed:
 *                      s_col = float [ceil(cols/128) x ceil(rows/128)]
 *        MX_1x32       32 rows down each column:
 *                      s_col = uint8 [cols x ceil(rows/32)]
 *        CHANNEL       s_col = float [cols]  (s_inv of each whole column)
 *        TENSOR_*      same scale as ROW (a plain transpose of the codes).
 *   scale, scale_inv, amax       : per-tensor recipes only (device floats).
 *        CURRENT: amax is float[FP8MI_AMAX_SLOTS]: amax[0] receives
 *                 max|x| (NaN if x holds a NaN); amax[1..] is scratch for
 *                 per-workgroup partial maxima (left holding them).  Writes
 *                 scale and scale_inv.
 *        DELAYED: reads *scale; amax is the accumulator
 *                 float[FP8MI_AMAX_SLOTS]: the step's amax is the largest
 *                 slot (NaN-dominant, comparing |x| bit patterns) and a cast
 *                 raises slots to cover max|x| of x.  The caller zeroes it
 *                 once; fp8_amax_history_update consumes and re-zeroes it.
 *                 Casts that share an accumulator must be ordered on one
 *                 stream.  scale_inv is not touched.
 *        CHANNEL: before the cast, the code outputs briefly hold per-tile
 *                 partial maxima inside their logical bytes and the scale
 *                 outputs hold the scales s; both are final on completion.
 *   nonfinite                    : optional (may be NULL) device int32; gets
 *        += the number of scale blocks whose amax was NaN/Inf (CURRENT,
 *        channel and block recipes; those blocks use s = 1, MX byte 0xFF).
 * x must not overlap any output.
 * Alignment: x, q_row, q_col 16-byte aligned; ld_x * sizeof(elem),
 * ld_q_row and ld_q_col multiples of 16 bytes.  Sizes: rows * ld_x *
 * sizeof(elem), rows * ld_q_row and cols * ld_q_col must fit in int64 (else
 * FP8MI_ERR_SHAPE); CHANNEL needs ceil(rows/128) * ceil(cols/128) < 2^31
 * (else FP8MI_ERR_UNSUPPORTED); the other recipes take any size.  rows == 0 or cols == 0 is
 * allowed (CURRENT then writes amax = 0, scale = scale_inv = 1).
 * Returns FP8MI_OK or an FP8MI_ERR_* code; nothing is launched on error. */
int fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                 int recipe, int fmt, int orient, int margin,
                 uint8_t* q_row, int64_t ld_q_row, void* s_row,
                 uint8_t* q_col, int64_t ld_q_col, void* s_col,
                 float* scale, float* scale_inv, float* amax, int32_t* nonfinite,
                 void* stream);

/* fp8_quantize_static_scratch -- fp8_quantize for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, checks, results and errors as
 * fp8_quantize, with one difference: TENSOR_CURRENT keeps the partial maxima
 * of its amax pass in a static device array of the library (1024 words =
 * 4 KB per GPU, allocated when the library is loaded and held until the
 * process ends) instead of amax[1 ..], so `amax` need hold only amax[0]
 * (one float).  The pass uses at most 1023 partials whatever the tensor's
 * size, so no size is refused for want of scratch.  TENSOR_DELAYED still
 * takes its float[FP8MI_AMAX_SLOTS] accumulator (caller-owned state, not
 * scratch).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams) race and must be ordered
 * by the caller; each call writes every slot it reads before reading it. */
int fp8_quantize_static_scratch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                int recipe, int fmt, int orient, int margin,
                                uint8_t* q_row, int64_t ld_q_row, void* s_row,
                                uint8_t* q_col, int64_t ld_q_col, void* s_col,
                                float* scale, float* scale_inv, float* amax, int32_t* nonfinite,
                                void* stream);

/* fp8_amax_history_update -- one delayed-scaling step.
 * [P1 sec. 2.1: amax history over the past steps (usually 200), scale from
 *  the maximum of the buffer; P2 sec. 3.3: interval 1 = every step, margin]
 *
 *   history  : float [len] ring, zero-initialised by the caller; head: int32.
 *   amax     : float[FP8MI_AMAX_SLOTS], the accumulator that fp8_quantize
 *              with TENSOR_DELAYED filled since the previous update; its
 *              largest slot is the step's amax a; every slot is reset to 0.
 *   If a is finite it is written to history[h] and head = (h + 1) % len,
 *   with h = *head reduced modulo len into [0, len); otherwise
 *   *nonfinite += 1 and nothing is pushed.  Then scale = s(max(history)), scale_inv = fl32(1 / scale).
 *   len in [1, 65536]; margin in [0, 64].  One workgroup; device state only. */
int fp8_amax_history_update(float* history, int32_t* head, int64_t len, float* amax, int fmt,
                            int margin, float* scale, float* scale_inv, int32_t* nonfinite,
                            void* stream);

/* fp8_gemm_scaled -- C = dequant(A) . dequant(B)^T, FP32 accumulation.
 * [P1 sec. 3.1: fprop Y = X W, dgrad dX = dY W^T, wgrad dW = X^T dY on
 *  quantized inputs with BF16/FP32 outputs; P3 Fig. 1 discussion: per-block
 *  scale factors are applied inside the GEMM]
 *
 *   layout   : FP8MI_LAYOUT_TN (the only layout built; any other value
 *              returns FP8MI_ERR_UNSUPPORTED before any launch):
 *   a [M x K] codes (fmt_a), lda; b [N x K] codes (fmt_b), ldb; both with
 *   the contraction index K contiguous.  c [M x N] (c_dtype), ldc.
 *   s_a, s_b : dequantisation scales laid out per `recipe` (see FP8MI_GEMM_*;
 *              grids are dense, row-major).  Block recipes scale K-block kb
 *              = k / 128 (MX: k / 32); 128x128 tiles of B are indexed
 *              [n / 128][k / 128].
 *   C[i][j] = sum_k deq(a[i][k]) * deq(b[j][k]) with deq = dec(code) * scale;
 *   block recipes accumulate each 128-deep K block in an FP32 partial and
 *   add scale_a * scale_b * partial to the FP32 accumulator.
 *   Uses:  fprop  a = X   [M x K], b = W   [N x K];
 *          dgrad  a = dY  [M x N], b = W^T [K x N]  (contraction over N);
 *          wgrad  a = dY^T[N x M], b = X^T [K x M]  (contraction over M).
 *   BLOCK_128x128_128x128 (both operands in 128x128 tiles) promotes each
 *   128-deep block with s_a[i / 128][kb] * s_b[j / 128][kb]; CHANNEL
 *   scales the FP32 result by s_a[i] * s_b[j] (the rows of a and b are the
 *   channels: a per-row scale of X and a per-output-channel scale of W).
 *   Non-finite inputs follow IEEE arithmetic: a NaN code (E4M3 0x7F/0xFF,
 *   E5M2 0x7D-0x7F/0xFD-0xFF), an E5M2 infinity (0x7C/0xFC) or an E8M0 NaN
 *   scale (0xFF) gives the NaN or infinity of the float64 reference.
 * Requirements: M, N, K >= 0; K % 16 == 0; a, b 16-byte aligned,
 * s_a, s_b 4-byte aligned (scale grids are read in aligned dwords; for MX
 * that may touch up to 3 bytes past a grid's last row, never used),
 * lda, ldb multiples of 16, K <= lda, ldb <= 4194304 and
 * ceil(M/256) * ceil(N/256) < 2^31 (else FP8MI_ERR_UNSUPPORTED); ldc >= N
 * with M * ldc * sizeof(c element) fitting in int64 (else FP8MI_ERR_SHAPE).
 * c must not overlap a, b or the scales.  K == 0 writes zeros.
 * Tolerance vs a float64 reference over the dequantized operands:
 * |C - C_ref| <= 2^-10 sum_k |a b| (+ 2^-8 |C_ref| for BF16 output). */
int fp8_gemm_scaled(const uint8_t* a, int fmt_a, const void* s_a, int64_t lda,
                    const uint8_t* b, int fmt_b, const void* s_b, int64_t ldb,
                    int recipe, int layout, int64_t M, int64_t N, int64_t K,
                    void* c, int c_dtype, int64_t ldc, void* stream);

/* fp8_bf16_gemm -- C = A . B^T with BF16 operands and FP32 accumulation:
 * the BF16 GEMM that FP8's speedup is measured against [P3 Fig. 1: FP8
 * GEMM throughput of each scaling strategy relative to BF16, over K].  It
 * is the fp8_gemm_scaled kernel with the BF16 matrix-core instruction in
 * place of the FP8 one: same tiles, data movement and epilogue.
 *
 *   a [M x K] BF16, lda; b [N x K] BF16, ldb (elements, K contiguous);
 *   c [M x N] (c_dtype), ldc.  C[i][j] = sum_k a[i][k] * b[j][k].
 * Requirements: M, N, K >= 0; K % 8 == 0; a, b 16-byte aligned, lda, ldb
 * multiples of 8, K <= lda, ldb <= 2097152 and ceil(M/256) * ceil(N/256)
 * < 2^31 (else FP8MI_ERR_UNSUPPORTED); ldc >= N, M * ldc * sizeof(c element)
 * fitting in int64.  K == 0 writes zeros.  Errors as for fp8_gemm_scaled.
 * Tolerance vs a float64 reference: as fp8_gemm_scaled. */
int fp8_bf16_gemm(const void* a, int64_t lda, const void* b, int64_t ldb,
                  int64_t M, int64_t N, int64_t K,
                  void* c, int c_dtype, int64_t ldc, void* stream);

/* Human-readable text of a status code; for FP8MI_ERR_HIP the text of the
 * last HIP error seen by this thread.  The string is owned by the library. */
const char* fp8_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8MI_H */
