/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for FP8 scaled
 * quantization (per-tensor current / delayed, 1x128 / 128x128 blocks,
 * 1x32 MX blocks with E8M0 scales) and the amax-history update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant with the HIP library: every value below is
 * re-derived here from the format definitions.
 *
 * Build: gcc -O2 -std=c99 -fno-fast-math -ffp-contract=off -fPIC -shared
 * (no FMA contraction, so every `a * b` and `a / b` on `float` is a single
 * IEEE-754 binary32 operation rounded to nearest-even).
 *
 * Sources (cited by page and section):
 *   [P1] "2025 technical guide: FP8 quantized training" (blog.gitcode.com),
 *        sec. 1.1 (bit layouts), 2.1 (per-tensor delayed / current scaling,
 *        200-step amax history), 2.2 (blockwise 1x128 / 128x128),
 *        2.3 (MXFP8 1x32 blocks, E8M0 scales), 3.1 (fprop/dgrad/wgrad).
 *   [P2] "From FP16 to FP8" (bjdmk.com.cn/news/5220490), sec. 1 (E5M2 range
 *        57344 .. 6.1e-5), sec. 2 (E5M2 bias 15, 2 mantissa bits),
 *        sec. 3.3 (DelayedScaling margin=0, interval=1).
 *   [P3] "Mastering FP8 LLM training" (nmedialink.com), strategy 1
 *        (delayed), 2 (current), 3 (sub-channel blocks), 4 (MXFP8).
 *   [P4] "FP8 training support" (bjdmk.com.cn/news/366077), section
 *        "Why FP8?" (E4M3 ~400 range for weights/activations, E5M2 for
 *        gradients, dynamic scaling maps the FP32 range onto FP8).
 *
 * Readings where the pages are silent:
 *   - E4M3 is OCP E4M3FN (max 448, subnormals, no Inf, NaN = S.1111.111);
 *     E5M2 is OCP E5M2 (max 57344, subnormals, Inf = S.11111.00).
 *   - Encoding is round-to-nearest, ties to the even code, saturating:
 *     |v| >= max (and +-Inf) gives +-max; NaN gives 0x7F; -0 stays 0x80.
 *   - Scale s = fl32(max / amax) * 2^-margin, applied as fl32(x * s)
 *     (two roundings); s_inv = fl32(1 / s) is what the GEMM consumes.
 *     amax == 0 -> s = 1; non-finite amax -> s = 1 and a flag; s = +Inf
 *     (tiny amax) -> FLT_MAX.
 *   - MX: E8M0 exponent e = ceil(log2(amax / max)), clamped to [-127, 127],
 *     stored as e + 127; amax == 0 -> 127; non-finite amax -> 0xFF.  The
 *     OCP specification's floor rule (e = floor(log2 amax) - emax) is a
 *     variant, selected per call.
 *   - Channel-wise scaling ("Mastering FP8 LLM training", Fig. 1 discussion:
 *     one scale per channel, i.e. per row or column) is block scaling with
 *     1 x cols blocks; it needs no code of its own here.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_E4M3 0
#define OR_E5M2 1

/* ------------------------------------------------------------------ */
/* Formats [P1 sec.1.1, P2 sec.1-2, P4 "Why FP8?"]                      */
/* ------------------------------------------------------------------ */

/* Value of an FP8 code, straight from the bit fields.
 * E4M3: sign = bit 7, exponent = bits 6..3 (bias 7), mantissa = bits 2..0.
 * E5M2: sign = bit 7, exponent = bits 6..2 (bias 15), mantissa = bits 1..0. */
double or_decode(int fmt, int code)
{
    int sign = (code >> 7) & 1;
    double v;
    if (fmt == OR_E4M3) {
        int e = (code >> 3) & 15, m = code & 7;
        if (e == 15 && m == 7)
            return NAN;
        if (e == 0)
            v = ldexp((double)m / 8.0, 1 - 7);           /* 0.m * 2^(1-bias) */
        else
            v = ldexp(1.0 + (double)m / 8.0, e - 7);     /* 1.m * 2^(e-bias) */
    } else {
        int e = (code >> 2) & 31, m = code & 3;
        if (e == 31)
            return m == 0 ? (sign ? -INFINITY : INFINITY) : NAN;
        if (e == 0)
            v = ldexp((double)m / 4.0, 1 - 15);
        else
            v = ldexp(1.0 + (double)m / 4.0, e - 15);
    }
    return sign ? -v : v;
}

/* Largest finite positive code: E4M3 S.1111.110 = 448, E5M2 S.11110.11 = 57344. */
int or_max_code(int fmt)
{
    return fmt == OR_E4M3 ? 0x7E : 0x7B;
}

double or_max_value(int fmt)
{
    return or_decode(fmt, or_max_code(fmt));
}

/* Table of decoded values, filled from or_decode on first use, so the
 * search below does not recompute the bit-field formula every probe. */
static double g_tab[2][256];
static int g_tab_ready[2];

static double grid(int fmt, int code)
{
    if (!g_tab_ready[fmt]) {
        for (int c = 0; c < 256; ++c)
            g_tab[fmt][c] = or_decode(fmt, c);
        g_tab_ready[fmt] = 1;
    }
    return g_tab[fmt][code];
}

/* Round v to the nearest value of the format's finite grid, ties to the
 * code whose lowest bit is 0, saturating at the largest finite value.
 * Plain search over the (monotone) table of non-negative finite values. */
int or_encode(int fmt, float v)
{
    if (isnan(v))
        return 0x7F;
    int sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    int top = or_max_code(fmt);
    if (a >= grid(fmt, top))
        return sign | top;
    /* invariant: grid(lo) <= a < grid(hi) */
    int lo = 0, hi = top;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (grid(fmt, mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double glo = grid(fmt, lo), ghi = grid(fmt, hi);
    double half = (glo + ghi) / 2.0; /* exact: both have few significant bits */
    int code;
    if (a < half)
        code = lo;
    else if (a > half)
        code = hi;
    else
        code = (lo % 2 == 0) ? lo : hi;
    return sign | code;
}

void or_encode_array(int fmt, const float* v, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)or_encode(fmt, v[i]);
}

void or_decode_array(int fmt, const uint8_t* c, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_decode(fmt, c[i]);
}

/* ------------------------------------------------------------------ */
/* Scale from amax [P1 sec.2.1, P2 sec.3.3 margin, P4 "Why FP8?"]       */
/* ------------------------------------------------------------------ */

/* s maps amax onto the format maximum; s_inv undoes it for the GEMM.
 * Returns 1 when amax was not finite (s falls back to 1). */
int or_scale_from_amax(int fmt, float amax, int margin, float* s_out, float* s_inv_out)
{
    float fmax = (float)or_max_value(fmt);
    float s;
    int flag = 0;
    if (!isfinite(amax)) {
        s = 1.0f;
        flag = 1;
    } else if (amax == 0.0f) {
        s = 1.0f;
    } else {
        s = fmax / amax;
        s = ldexpf(s, -margin);
        if (isinf(s))
            s = FLT_MAX;
    }
    *s_out = s;
    *s_inv_out = 1.0f / s;
    return flag;
}

/* ------------------------------------------------------------------ */
/* amax reduction [P1 sec.2.1-2.3]                                     */
/* ------------------------------------------------------------------ */

/* max |x| over rows [r0,r1) x cols [c0,c1) of a row-major matrix with
 * leading dimension ld.  A NaN anywhere makes the result NaN. */
float or_amax_block(const float* x, int64_t ld, int64_t r0, int64_t r1, int64_t c0, int64_t c1)
{
    float m = 0.0f;
    int saw_nan = 0;
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = c0; j < c1; ++j) {
            float a = fabsf(x[i * ld + j]);
            if (isnan(a))
                saw_nan = 1;
            else if (a > m)
                m = a;
        }
    return saw_nan ? NAN : m;
}

/* ------------------------------------------------------------------ */
/* Cast with a given scale: q = enc(fl32(x * s))                       */
/* ------------------------------------------------------------------ */

void or_cast_block(int fmt, const float* x, int64_t ld, int64_t r0, int64_t r1, int64_t c0,
                   int64_t c1, float s, uint8_t* q, int64_t ldq)
{
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t j = c0; j < c1; ++j) {
            float p = x[i * ld + j] * s;
            q[i * ldq + j] = (uint8_t)or_encode(fmt, p);
        }
}

/* Per-tensor current scaling [P1 sec.2.1, P3 strategy 2]: amax of this
 * tensor, then s, then the cast.  Returns the non-finite flag. */
int or_quantize_current(int fmt, const float* x, int64_t rows, int64_t cols, int margin,
                        uint8_t* q, float* s_out, float* s_inv_out, float* amax_out)
{
    float amax = or_amax_block(x, cols, 0, rows, 0, cols);
    float s, s_inv;
    int flag = or_scale_from_amax(fmt, amax, margin, &s, &s_inv);
    or_cast_block(fmt, x, cols, 0, rows, 0, cols, s, q, cols);
    *s_out = s;
    *s_inv_out = s_inv;
    *amax_out = amax;
    return flag;
}

/* Per-tensor delayed scaling, cast half [P1 sec.2.1, P3 strategy 1]: the
 * cast uses the scale carried over from earlier steps; this tensor's amax
 * is returned for the history update. */
void or_quantize_delayed(int fmt, const float* x, int64_t rows, int64_t cols, float s,
                         uint8_t* q, float* amax_out)
{
    *amax_out = or_amax_block(x, cols, 0, rows, 0, cols);
    or_cast_block(fmt, x, cols, 0, rows, 0, cols, s, q, cols);
}

/* Block scaling [P1 sec.2.2, P3 strategy 3]: every br x bc block (edge
 * blocks may be partial) is scaled as its own tensor with current scaling.
 * 1x128 rows: (1,128); 128 tokens down a column: (128,1); weights (128,128).
 * s_inv is a row-major grid of ceil(rows/br) x ceil(cols/bc) FP32 values.
 * Returns the number of blocks whose amax was not finite. */
int64_t or_quantize_blocks(int fmt, const float* x, int64_t rows, int64_t cols, int64_t br,
                           int64_t bc, int margin, uint8_t* q, float* s_inv)
{
    int64_t gr = (rows + br - 1) / br, gc = (cols + bc - 1) / bc, bad = 0;
    for (int64_t bi = 0; bi < gr; ++bi)
        for (int64_t bj = 0; bj < gc; ++bj) {
            int64_t r0 = bi * br, r1 = r0 + br < rows ? r0 + br : rows;
            int64_t c0 = bj * bc, c1 = c0 + bc < cols ? c0 + bc : cols;
            float amax = or_amax_block(x, cols, r0, r1, c0, c1);
            float s, si;
            bad += or_scale_from_amax(fmt, amax, margin, &s, &si);
            or_cast_block(fmt, x, cols, r0, r1, c0, c1, s, q, cols);
            s_inv[bi * gc + bj] = si;
        }
    return bad;
}

/* ------------------------------------------------------------------ */
/* MX blocks with E8M0 scales [P1 sec.2.3, P3 strategy 4]               */
/* ------------------------------------------------------------------ */

/* E8M0 byte for a block amax: the smallest power of two 2^e with
 * amax * 2^-e <= max (so no element of the block saturates).  Writing
 * amax = f * 2^E with f in [1,2) and max = 1.75 * 2^emax (emax = 8 for
 * E4M3, 15 for E5M2): e = E - emax, plus one when f > 1.75. */
int or_mx_scale_byte(int fmt, float amax)
{
    if (!isfinite(amax))
        return 0xFF;
    if (amax == 0.0f)
        return 127;
    int E2;
    double f = frexp((double)amax, &E2); /* amax = f * 2^E2, f in [0.5, 1) */
    f *= 2.0;
    E2 -= 1; /* now f in [1, 2) */
    int emax = fmt == OR_E4M3 ? 8 : 15;
    int e = E2 - emax + (f > 1.75 ? 1 : 0);
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e + 127;
}

/* The OCP microscaling specification's rule, kept beside the one above as
 * a variant: the shared exponent is floor(log2(amax)) - emax, i.e. e = E -
 * emax for every f, so a block whose largest element has f > 1.75 saturates
 * that element to max instead of taking the next power of two.  Zero and
 * non-finite amax as above. */
int or_mx_scale_byte_floor(int fmt, float amax)
{
    if (!isfinite(amax))
        return 0xFF;
    if (amax == 0.0f)
        return 127;
    int E2;
    frexp((double)amax, &E2); /* amax = f * 2^E2, f in [0.5, 1) */
    int e = (E2 - 1) - (fmt == OR_E4M3 ? 8 : 15);
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e + 127;
}

/* 2^(byte - 127) as the dequantisation scale of an E8M0 byte; NaN for 0xFF. */
double or_e8m0_value(int byte)
{
    if (byte == 0xFF)
        return NAN;
    return ldexp(1.0, byte - 127);
}

/* MX quantize: blocks of br x bc (1x32 along a row or 32x1 down a column).
 * Elements are enc(fl32(x * 2^-e)); a non-finite block amax gives scale
 * byte 0xFF and elements enc(x). */
int64_t or_quantize_mx_rule(int fmt, const float* x, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                            int floor_rule, uint8_t* q, uint8_t* scale_bytes)
{
    int64_t gr = (rows + br - 1) / br, gc = (cols + bc - 1) / bc, bad = 0;
    for (int64_t bi = 0; bi < gr; ++bi)
        for (int64_t bj = 0; bj < gc; ++bj) {
            int64_t r0 = bi * br, r1 = r0 + br < rows ? r0 + br : rows;
            int64_t c0 = bj * bc, c1 = c0 + bc < cols ? c0 + bc : cols;
            float amax = or_amax_block(x, cols, r0, r1, c0, c1);
            int byte = floor_rule ? or_mx_scale_byte_floor(fmt, amax) : or_mx_scale_byte(fmt, amax);
            float s = 1.0f;
            if (byte == 0xFF)
                bad += 1;
            else
                s = ldexpf(1.0f, 127 - byte);
            or_cast_block(fmt, x, cols, r0, r1, c0, c1, s, q, cols);
            scale_bytes[bi * gc + bj] = (uint8_t)byte;
        }
    return bad;
}

int64_t or_quantize_mx(int fmt, const float* x, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                       uint8_t* q, uint8_t* scale_bytes)
{
    return or_quantize_mx_rule(fmt, x, rows, cols, br, bc, 0, q, scale_bytes);
}

/* ------------------------------------------------------------------ */
/* amax history [P1 sec.2.1 "past steps, usually 200, take the max";    */
/* P2 sec.3.3 interval=1 -> update every step]                          */
/* ------------------------------------------------------------------ */

/* One step: push a finite amax into the ring (a non-finite one is not
 * pushed; the counter records it), then the next scale from the ring max. */
int or_history_update(float* ring, int32_t* head, int len, float amax, int fmt, int margin,
                      float* s_out, float* s_inv_out, int32_t* nonfinite)
{
    int pushed = 0;
    if (isfinite(amax)) {
        /* a stored head outside [0, len) (state saved with another length)
           is taken modulo len, the reading the C ABI documents */
        int h = *head % len;
        if (h < 0)
            h += len;
        ring[h] = amax;
        *head = (h + 1) % len;
        pushed = 1;
    } else {
        *nonfinite += 1;
    }
    float m = 0.0f;
    for (int i = 0; i < len; ++i)
        if (ring[i] > m)
            m = ring[i];
    or_scale_from_amax(fmt, m, margin, s_out, s_inv_out);
    return pushed;
}
