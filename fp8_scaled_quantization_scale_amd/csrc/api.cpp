// api.cpp -- the C ABI declared in include/fp8mi.h: host-side argument
// validation (no HIP call is made before it passes) and dispatch to the
// kernel launchers.  The library allocates nothing and keeps no state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>

#include "fp8mi.h"
#include "launch.hpp"

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FP8MI_OK;
  std::snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return FP8MI_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// rows x ld elements of esize bytes span a byte range that fits in int64 (no
// array that large can exist; checking first keeps every later size
// computation here and in the launchers free of overflow)
bool extent_ok(int64_t rows, int64_t ld, int64_t esize) {
  int64_t n = 0;
  return !__builtin_mul_overflow(rows, ld, &n) && !__builtin_mul_overflow(n, esize, &n);
}

// the persistent GEMM grid numbers its 256 x 256 output tiles with 32-bit ints
bool tile_count_ok(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256) <= 0x7FFFFFFFLL; }

int check_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int recipe,
                   int fmt, int orient, int margin, const uint8_t* q_row, int64_t ld_q_row,
                   const void* s_row, const uint8_t* q_col, int64_t ld_q_col, const void* s_col,
                   const float* scale, const float* scale_inv, const float* amax) {
  if (x_dtype != FP8MI_IN_BF16 && x_dtype != FP8MI_IN_FP32) return FP8MI_ERR_ENUM;
  if (recipe < FP8MI_TENSOR_CURRENT || recipe > FP8MI_MX_1x32_OCP) return FP8MI_ERR_ENUM;
  if (fmt != FP8MI_E4M3 && fmt != FP8MI_E5M2) return FP8MI_ERR_ENUM;
  if (orient != FP8MI_ROW && orient != FP8MI_COL && orient != FP8MI_ROW_AND_COL) return FP8MI_ERR_ENUM;
  if (rows < 0 || cols < 0 || margin < 0 || margin > 64) return FP8MI_ERR_SHAPE;
  const bool row = orient & FP8MI_ROW, col = orient & FP8MI_COL;
  const bool tensor = recipe == FP8MI_TENSOR_CURRENT || recipe == FP8MI_TENSOR_DELAYED;
  if (tensor) {
    if (!amax) return FP8MI_ERR_NULL;
    if (!scale) return FP8MI_ERR_NULL;
    if (recipe == FP8MI_TENSOR_CURRENT && !scale_inv) return FP8MI_ERR_NULL;
  }
  const bool empty = rows == 0 || cols == 0;
  if (empty) return FP8MI_OK;
  if (!x) return FP8MI_ERR_NULL;
  if (row && (!q_row || (!tensor && !s_row))) return FP8MI_ERR_NULL;
  if (col && (!q_col || (!tensor && !s_col))) return FP8MI_ERR_NULL;
  if (ld_x < cols) return FP8MI_ERR_SHAPE;
  if (row && ld_q_row < cols) return FP8MI_ERR_SHAPE;
  if (col && ld_q_col < rows) return FP8MI_ERR_SHAPE;
  const int64_t esize = x_dtype == FP8MI_IN_BF16 ? 2 : 4;
  if (!extent_ok(rows, ld_x, esize)) return FP8MI_ERR_SHAPE;
  if (row && !extent_ok(rows, ld_q_row, 1)) return FP8MI_ERR_SHAPE;
  if (col && !extent_ok(cols, ld_q_col, 1)) return FP8MI_ERR_SHAPE;
  if (!aligned16(x) || (ld_x * esize) % 16) return FP8MI_ERR_ALIGN;
  if (row && (!aligned16(q_row) || ld_q_row % 16)) return FP8MI_ERR_ALIGN;
  if (col && (!aligned16(q_col) || ld_q_col % 16)) return FP8MI_ERR_ALIGN;
  // channel scaling launches one workgroup per tile on a 1-D grid
  if (recipe == FP8MI_CHANNEL && ((rows + 127) / 128) * ((cols + 127) / 128) > 0x7FFFFFFF)
    return FP8MI_ERR_UNSUPPORTED;
  return FP8MI_OK;
}

int check_gemm(const uint8_t* a, int fmt_a, const void* s_a, int64_t lda, const uint8_t* b, int fmt_b,
               const void* s_b, int64_t ldb, int recipe, int layout, int64_t M, int64_t N, int64_t K,
               const void* c, int c_dtype, int64_t ldc) {
  if (layout != FP8MI_LAYOUT_TN) return FP8MI_ERR_UNSUPPORTED;
  if (fmt_a != FP8MI_E4M3 && fmt_a != FP8MI_E5M2) return FP8MI_ERR_ENUM;
  if (fmt_b != FP8MI_E4M3 && fmt_b != FP8MI_E5M2) return FP8MI_ERR_ENUM;
  if (recipe < FP8MI_GEMM_TENSOR || recipe > FP8MI_GEMM_CHANNEL) return FP8MI_ERR_ENUM;
  if (c_dtype != FP8MI_OUT_BF16 && c_dtype != FP8MI_OUT_FP32) return FP8MI_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0) return FP8MI_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8MI_OK;
  if (!c) return FP8MI_ERR_NULL;
  if (ldc < N) return FP8MI_ERR_SHAPE;
  if (!extent_ok(M, ldc, c_dtype == FP8MI_OUT_FP32 ? 4 : 2)) return FP8MI_ERR_SHAPE;
  if (K > 0) {
    if (!a || !b || !s_a || !s_b) return FP8MI_ERR_NULL;
    if (K % 16) return FP8MI_ERR_SHAPE;
    if (lda < K || ldb < K) return FP8MI_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || lda % 16 || ldb % 16) return FP8MI_ERR_ALIGN;
    // scale grids are read in whole aligned dwords (MX rows' E8M0 bytes too)
    if (((uintptr_t)s_a & 3u) || ((uintptr_t)s_b & 3u)) return FP8MI_ERR_ALIGN;
  }
  if (M > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > 0x7FFFFFFFLL) return FP8MI_ERR_UNSUPPORTED;
  // operand panels are addressed with 32-bit buffer offsets
  if (K > 0 && (lda > (1LL << 22) || ldb > (1LL << 22))) return FP8MI_ERR_UNSUPPORTED;
  if (!tile_count_ok(M, N)) return FP8MI_ERR_UNSUPPORTED;
  return FP8MI_OK;
}

}  // namespace

extern "C" {

int fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int recipe,
                 int fmt, int orient, int margin, uint8_t* q_row, int64_t ld_q_row, void* s_row,
                 uint8_t* q_col, int64_t ld_q_col, void* s_col, float* scale, float* scale_inv,
                 float* amax, int32_t* nonfinite, void* stream) {
  int st = check_quantize(x, x_dtype, rows, cols, ld_x, recipe, fmt, orient, margin, q_row, ld_q_row,
                          s_row, q_col, ld_q_col, s_col, scale, scale_inv, amax);
  if (st != FP8MI_OK) return st;
  if ((rows == 0 || cols == 0) && recipe != FP8MI_TENSOR_CURRENT) return FP8MI_OK;
  fp8mi::QuantParams p{x,      x_dtype,  rows,  cols,  ld_x,     recipe, fmt,      orient, margin,
                       q_row,  ld_q_row, s_row, q_col, ld_q_col, s_col,  scale,    scale_inv,
                       amax,   nonfinite};
  return hip_status(fp8mi::launch_quantize(p, (hipStream_t)stream));
}

int fp8_quantize_static_scratch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, int recipe,
                                int fmt, int orient, int margin, uint8_t* q_row, int64_t ld_q_row, void* s_row,
                                uint8_t* q_col, int64_t ld_q_col, void* s_col, float* scale, float* scale_inv,
                                float* amax, int32_t* nonfinite, void* stream) {
  int st = check_quantize(x, x_dtype, rows, cols, ld_x, recipe, fmt, orient, margin, q_row, ld_q_row,
                          s_row, q_col, ld_q_col, s_col, scale, scale_inv, amax);
  if (st != FP8MI_OK) return st;
  if ((rows == 0 || cols == 0) && recipe != FP8MI_TENSOR_CURRENT) return FP8MI_OK;
  fp8mi::QuantParams p{x,      x_dtype,  rows,  cols,  ld_x,     recipe, fmt,      orient, margin,
                       q_row,  ld_q_row, s_row, q_col, ld_q_col, s_col,  scale,    scale_inv,
                       amax,   nonfinite};
  return hip_status(fp8mi::launch_quantize_static_scratch(p, (hipStream_t)stream));
}

int fp8_amax_history_update(float* history, int32_t* head, int64_t len, float* amax, int fmt, int margin,
                            float* scale, float* scale_inv, int32_t* nonfinite, void* stream) {
  if (fmt != FP8MI_E4M3 && fmt != FP8MI_E5M2) return FP8MI_ERR_ENUM;
  if (!history || !head || !amax || !scale || !scale_inv) return FP8MI_ERR_NULL;
  if (len < 1 || len > 65536 || margin < 0 || margin > 64) return FP8MI_ERR_SHAPE;
  return hip_status(fp8mi::launch_history(history, head, (int)len, amax, fmt, margin, scale, scale_inv,
                                          nonfinite, (hipStream_t)stream));
}

int fp8_gemm_scaled(const uint8_t* a, int fmt_a, const void* s_a, int64_t lda, const uint8_t* b, int fmt_b,
                    const void* s_b, int64_t ldb, int recipe, int layout, int64_t M, int64_t N, int64_t K,
                    void* c, int c_dtype, int64_t ldc, void* stream) {
  int st = check_gemm(a, fmt_a, s_a, lda, b, fmt_b, s_b, ldb, recipe, layout, M, N, K, c, c_dtype, ldc);
  if (st != FP8MI_OK) return st;
  if (M == 0 || N == 0) return FP8MI_OK;
  fp8mi::GemmParams p{a, fmt_a, s_a, lda, b, fmt_b, s_b, ldb, recipe, M, N, K, c, c_dtype, ldc};
  return hip_status(fp8mi::launch_gemm(p, (hipStream_t)stream));
}

int fp8_bf16_gemm(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t M, int64_t N, int64_t K,
                  void* c, int c_dtype, int64_t ldc, void* stream) {
  if (c_dtype != FP8MI_OUT_BF16 && c_dtype != FP8MI_OUT_FP32) return FP8MI_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0) return FP8MI_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8MI_OK;
  if (!c) return FP8MI_ERR_NULL;
  if (ldc < N) return FP8MI_ERR_SHAPE;
  if (!extent_ok(M, ldc, c_dtype == FP8MI_OUT_FP32 ? 4 : 2)) return FP8MI_ERR_SHAPE;
  if (K > 0) {
    if (!a || !b) return FP8MI_ERR_NULL;
    if (K % 8) return FP8MI_ERR_SHAPE;
    if (lda < K || ldb < K) return FP8MI_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(b) || lda % 8 || ldb % 8) return FP8MI_ERR_ALIGN;
  }
  if (M > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > 0x3FFFFFFFLL) return FP8MI_ERR_UNSUPPORTED;
  if (K > 0 && (lda > (1LL << 21) || ldb > (1LL << 21))) return FP8MI_ERR_UNSUPPORTED;
  if (!tile_count_ok(M, N)) return FP8MI_ERR_UNSUPPORTED;
  fp8mi::GemmParams p{reinterpret_cast<const uint8_t*>(a), 0, nullptr, lda, reinterpret_cast<const uint8_t*>(b), 0,
                      nullptr, ldb, FP8MI_GEMM_TENSOR, M, N, K, c, c_dtype, ldc};
  return hip_status(fp8mi::launch_gemm_bf16(p, (hipStream_t)stream));
}

const char* fp8_status_string(int status) {
  switch (status) {
    case FP8MI_OK: return "ok";
    case FP8MI_ERR_NULL: return "a required pointer is NULL";
    case FP8MI_ERR_ENUM: return "unknown recipe, format, orientation or dtype value";
    case FP8MI_ERR_SHAPE: return "bad size, leading dimension or margin";
    case FP8MI_ERR_UNSUPPORTED: return "valid arguments, but this combination is not supported";
    case FP8MI_ERR_ALIGN: return "pointer or leading dimension breaks its alignment (16 bytes; GEMM scales 4)";
    case FP8MI_ERR_HIP: return g_hip_msg;
  }
  return "unknown status";
}

int fp8_version(void) { return 500; }

}  // extern "C"
