/*
 * Host driver for the C oracle (oracle/oracle.c), built together with it
 * under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize.py.  It walks every entry point over the edge inputs
 * the quantize path meets: every code of both formats, zero, subnormal,
 * huge and non-finite amax, ragged blocks (1x1 .. 3x130 shapes, blocks
 * larger than the tensor), MX blocks under both exponent rules, and an
 * amax history whose head starts out of range.  The sanitizers check the
 * memory accesses and the integer arithmetic; the few value checks here
 * only guard against a silently skipped call.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double or_decode(int fmt, int code);
int or_max_code(int fmt);
double or_max_value(int fmt);
int or_encode(int fmt, float v);
void or_encode_array(int fmt, const float* v, uint8_t* out, int64_t n);
void or_decode_array(int fmt, const uint8_t* c, double* out, int64_t n);
int or_scale_from_amax(int fmt, float amax, int margin, float* s_out, float* s_inv_out);
float or_amax_block(const float* x, int64_t ld, int64_t r0, int64_t r1, int64_t c0, int64_t c1);
void or_cast_block(int fmt, const float* x, int64_t ld, int64_t r0, int64_t r1, int64_t c0, int64_t c1, float s,
                   uint8_t* q, int64_t ldq);
int or_quantize_current(int fmt, const float* x, int64_t rows, int64_t cols, int margin, uint8_t* q, float* s_out,
                        float* s_inv_out, float* amax_out);
void or_quantize_delayed(int fmt, const float* x, int64_t rows, int64_t cols, float s, uint8_t* q, float* amax_out);
int64_t or_quantize_blocks(int fmt, const float* x, int64_t rows, int64_t cols, int64_t br, int64_t bc, int margin,
                           uint8_t* q, float* s_inv);
int or_mx_scale_byte(int fmt, float amax);
int or_mx_scale_byte_floor(int fmt, float amax);
double or_e8m0_value(int byte);
int64_t or_quantize_mx_rule(int fmt, const float* x, int64_t rows, int64_t cols, int64_t br, int64_t bc,
                            int floor_rule, uint8_t* q, uint8_t* scale_bytes);
int64_t or_quantize_mx(int fmt, const float* x, int64_t rows, int64_t cols, int64_t br, int64_t bc, uint8_t* q,
                       uint8_t* scale_bytes);
int or_history_update(float* ring, int32_t* head, int len, float amax, int fmt, int margin, float* s_out,
                      float* s_inv_out, int32_t* nonfinite);

static int failures = 0;
static void check(int ok, const char* what) {
    if (!ok) {
        ++failures;
        printf("FAIL: %s\n", what);
    }
}

/* exactly-sized heap buffers, so that AddressSanitizer sees any overrun */
static float* fbuf(int64_t n) { return (float*)malloc((size_t)(n ? n : 1) * sizeof(float)); }
static uint8_t* bbuf(int64_t n) { return (uint8_t*)malloc((size_t)(n ? n : 1)); }

static float edge_value(int i) {
    static const float v[] = {0.0f, -0.0f, 1.0f, -1.5f, 448.0f, 449.0f, 57344.0f, 1e30f, 1e-45f, 1e-40f,
                              1.17549435e-38f, 3.0e-8f, 6.1e-5f, INFINITY, -INFINITY, NAN};
    return v[i % (int)(sizeof(v) / sizeof(v[0]))];
}

int main(void) {
    const int fmts[2] = {0, 1};
    for (int f = 0; f < 2; ++f) {
        int fmt = fmts[f];
        /* every code decodes; every decoded finite value re-encodes */
        for (int c = 0; c < 256; ++c) {
            double d = or_decode(fmt, c);
            if (isfinite(d)) check(or_decode(fmt, or_encode(fmt, (float)d)) == d || d == 0.0, "decode/encode round trip");
        }
        check(or_max_code(fmt) > 0 && or_max_value(fmt) > 0.0, "format maximum");
        /* scale derivation over edge amax values and margins */
        for (int i = 0; i < 16; ++i)
            for (int m = 0; m <= 64; m += 16) {
                float s = 0.0f, si = 0.0f;
                or_scale_from_amax(fmt, fabsf(edge_value(i)), m, &s, &si);
                /* (s may underflow to 0 for a huge amax under a large margin) */
                check(s >= 0.0f && !isnan(si), "scale not NaN");
                (void)or_mx_scale_byte(fmt, fabsf(edge_value(i)));
                (void)or_mx_scale_byte_floor(fmt, fabsf(edge_value(i)));
            }
        for (int b = 0; b < 256; ++b) (void)or_e8m0_value(b);
        /* arrays and blocks over ragged shapes, blocks larger than the tensor */
        const int64_t shapes[][2] = {{1, 1}, {1, 130}, {3, 1}, {3, 130}, {2, 33}, {129, 3}};
        const int64_t blocks[][2] = {{1, 128}, {128, 128}, {128, 1}, {1, 32}, {32, 1}, {1, 1}};
        for (size_t si = 0; si < sizeof(shapes) / sizeof(shapes[0]); ++si) {
            int64_t r = shapes[si][0], c = shapes[si][1], n = r * c;
            float* x = fbuf(n);
            uint8_t* q = bbuf(n);
            double* d = (double*)malloc((size_t)n * sizeof(double));
            for (int64_t k = 0; k < n; ++k) x[k] = edge_value((int)k) * (float)(k % 7 + 1);
            or_encode_array(fmt, x, q, n);
            or_decode_array(fmt, q, d, n);
            float s = 0, si2 = 0, am = 0;
            or_quantize_current(fmt, x, r, c, 0, q, &s, &si2, &am);
            or_quantize_delayed(fmt, x, r, c, 1.0f, q, &am);
            (void)or_amax_block(x, c, 0, r, 0, c);
            or_cast_block(fmt, x, c, 0, r, 0, c, 0.5f, q, c);
            for (size_t bi = 0; bi < sizeof(blocks) / sizeof(blocks[0]); ++bi) {
                int64_t br = blocks[bi][0], bc = blocks[bi][1];
                int64_t nb = ((r + br - 1) / br) * ((c + bc - 1) / bc);
                float* sinv = fbuf(nb);
                uint8_t* sb = bbuf(nb);
                (void)or_quantize_blocks(fmt, x, r, c, br, bc, 0, q, sinv);
                (void)or_quantize_mx(fmt, x, r, c, br, bc, q, sb);
                (void)or_quantize_mx_rule(fmt, x, r, c, br, bc, 1, q, sb);
                free(sinv);
                free(sb);
            }
            free(x);
            free(q);
            free(d);
        }
        /* amax history: a 200-step window filled past its edge, non-finite
           amax skipped, and heads outside [0, len) reduced into range */
        for (int len = 1; len <= 200; len += 199) {
            float* ring = fbuf(len);
            memset(ring, 0, (size_t)len * sizeof(float));
            const int32_t heads[] = {0, len - 1, len, -1, 1000003, -1000003};
            for (size_t hi = 0; hi < sizeof(heads) / sizeof(heads[0]); ++hi) {
                int32_t head = heads[hi], nonfinite = 0;
                for (int step = 0; step < 450; ++step) {
                    float s = 0, si = 0;
                    (void)or_history_update(ring, &head, len, edge_value(step), fmt, 0, &s, &si, &nonfinite);
                    check(head >= 0 && head < len, "history head in range");
                }
            }
            free(ring);
        }
    }
    if (failures) {
        printf("%d failure(s)\n", failures);
        return 1;
    }
    printf("oracle ok\n");
    return 0;
}
