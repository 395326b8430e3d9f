// Host-only driver for the C ABI's argument validation (api.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize.py.
// The kernel launchers are replaced by stubs that record what reached them,
// so every call below runs the library's own validation code on the host
// and nothing else; no GPU and no HIP runtime is involved.
#include <stdint.h>
#include <stdio.h>

#include <limits>

#include "fp8mi.h"
#include "launch.hpp"

namespace {
int g_launches = 0;
fp8mi::QuantParams g_q;
fp8mi::GemmParams g_g;
int g_failures = 0;

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    ++g_failures;
    printf("FAIL line %d: %s -> %d, expected %d\n", line, what, got, want);
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// 16-byte-aligned stand-ins for device pointers: validation never
// dereferences them, and the stub launchers do not either
alignas(64) unsigned char g_buf[4096];
void* const P = g_buf;
void* const P8 = g_buf + 8;
void* const P2 = g_buf + 2;
constexpr int64_t kMax = std::numeric_limits<int64_t>::max();
constexpr int64_t kMin = std::numeric_limits<int64_t>::min();
}  // namespace

namespace fp8mi {
hipError_t launch_quantize(const QuantParams& p, hipStream_t) {
  ++g_launches;
  g_q = p;
  return hipSuccess;
}
hipError_t launch_quantize_static_scratch(const QuantParams& p, hipStream_t) {
  ++g_launches;
  g_q = p;
  return hipSuccess;
}
hipError_t launch_empty_scale(float*, float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_history(float*, int32_t*, int, float*, int, int, float*, float*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gemm(const GemmParams& p, hipStream_t) {
  ++g_launches;
  g_g = p;
  return hipSuccess;
}
hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t) {
  ++g_launches;
  g_g = p;
  return hipSuccess;
}
}  // namespace fp8mi

// the one runtime call api.cpp makes (error text of a failed launch)
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace {

int quant(int64_t rows, int64_t cols, int64_t ld_x, int recipe, int orient, int64_t ld_q_row, int64_t ld_q_col,
          int x_dtype = FP8MI_IN_BF16, const void* x = P, int margin = 0) {
  float* f = static_cast<float*>(P);
  return fp8_quantize(x, x_dtype, rows, cols, ld_x, recipe, FP8MI_E4M3, orient, margin, static_cast<uint8_t*>(P),
                      ld_q_row, P, static_cast<uint8_t*>(P), ld_q_col, P, f, f, f, nullptr, nullptr);
}

int gemm(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int recipe = FP8MI_GEMM_TENSOR,
         const void* s_a = P, int c_dtype = FP8MI_OUT_BF16) {
  const uint8_t* u = static_cast<const uint8_t*>(P);
  return fp8_gemm_scaled(u, FP8MI_E4M3, s_a, lda, u, FP8MI_E4M3, P, ldb, recipe, FP8MI_LAYOUT_TN, M, N, K, P,
                         c_dtype, ldc, nullptr);
}

}  // namespace

int main() {
  // ---- quantize: ordinary calls reach the launcher with their arguments
  int before = g_launches;
  EXPECT(quant(256, 384, 384, FP8MI_BLOCK_1x128, FP8MI_ROW_AND_COL, 384, 256), FP8MI_OK);
  EXPECT(g_launches - before, 1);
  EXPECT((int)(g_q.rows == 256 && g_q.cols == 384 && g_q.ld_x == 384 && g_q.ld_q_col == 256), 1);
  EXPECT(quant(0, 384, 384, FP8MI_BLOCK_1x128, FP8MI_ROW, 384, 0), FP8MI_OK);  // empty: no launch
  EXPECT(g_launches - before, 1);
  // bad enums, sizes, pointers and alignment
  EXPECT(quant(256, 384, 384, 99, FP8MI_ROW, 384, 0), FP8MI_ERR_ENUM);
  EXPECT(quant(256, 384, 384, FP8MI_BLOCK_1x128, 7, 384, 0), FP8MI_ERR_ENUM);
  EXPECT(quant(-1, 384, 384, FP8MI_BLOCK_1x128, FP8MI_ROW, 384, 0), FP8MI_ERR_SHAPE);
  EXPECT(quant(256, 384, 383, FP8MI_BLOCK_1x128, FP8MI_ROW, 384, 0), FP8MI_ERR_SHAPE);
  EXPECT(quant(256, 384, 384, FP8MI_BLOCK_1x128, FP8MI_ROW, 384, 0, FP8MI_IN_BF16, nullptr), FP8MI_ERR_NULL);
  EXPECT(quant(256, 384, 384, FP8MI_BLOCK_1x128, FP8MI_ROW, 384, 0, FP8MI_IN_BF16, P8), FP8MI_ERR_ALIGN);
  EXPECT(quant(256, 384, 384, FP8MI_BLOCK_1x128, FP8MI_ROW, 384, 0, FP8MI_IN_BF16, P, 65), FP8MI_ERR_SHAPE);
  // extreme sizes: refused, with no overflow on the way (UBSan checks that)
  EXPECT(quant(kMax, kMax, kMax, FP8MI_BLOCK_1x128, FP8MI_ROW_AND_COL, kMax, kMax), FP8MI_ERR_SHAPE);
  EXPECT(quant(kMax, kMax, kMax, FP8MI_CHANNEL, FP8MI_ROW, kMax, kMax), FP8MI_ERR_SHAPE);
  EXPECT(quant(kMax, 128, kMax, FP8MI_TENSOR_CURRENT, FP8MI_ROW, kMax, 0, FP8MI_IN_FP32), FP8MI_ERR_SHAPE);
  EXPECT(quant(1, 128, kMax / 2 + 1, FP8MI_BLOCK_1x128, FP8MI_ROW, 128, 0), FP8MI_ERR_SHAPE);
  EXPECT(quant(1LL << 40, 1LL << 40, 1LL << 40, FP8MI_CHANNEL, FP8MI_COL, 0, 1LL << 40), FP8MI_ERR_SHAPE);
  EXPECT(quant(kMin, 1, 1, FP8MI_BLOCK_1x128, FP8MI_ROW, 1, 0), FP8MI_ERR_SHAPE);
  EXPECT(fp8_quantize_static_scratch(P, FP8MI_IN_BF16, kMax, kMax, kMax, FP8MI_TENSOR_CURRENT, FP8MI_E4M3,
                                     FP8MI_ROW, 0, static_cast<uint8_t*>(P), kMax, nullptr, nullptr, 0, nullptr,
                                     static_cast<float*>(P), static_cast<float*>(P), static_cast<float*>(P),
                                     nullptr, nullptr),
         FP8MI_ERR_SHAPE);

  // ---- history
  float* f = static_cast<float*>(P);
  EXPECT(fp8_amax_history_update(f, static_cast<int32_t*>(P), 200, f, FP8MI_E4M3, 0, f, f, nullptr, nullptr),
         FP8MI_OK);
  EXPECT(fp8_amax_history_update(f, static_cast<int32_t*>(P), kMax, f, FP8MI_E4M3, 0, f, f, nullptr, nullptr),
         FP8MI_ERR_SHAPE);
  EXPECT(fp8_amax_history_update(f, static_cast<int32_t*>(P), kMin, f, FP8MI_E4M3, 0, f, f, nullptr, nullptr),
         FP8MI_ERR_SHAPE);

  // ---- scaled GEMM
  before = g_launches;
  EXPECT(gemm(300, 200, 256, 256, 256, 200), FP8MI_OK);
  EXPECT(g_launches - before, 1);
  EXPECT((int)(g_g.M == 300 && g_g.N == 200 && g_g.K == 256 && g_g.ldc == 200), 1);
  EXPECT(gemm(300, 200, 256, 256, 256, 200, FP8MI_GEMM_MX_1x32, P2), FP8MI_ERR_ALIGN);
  EXPECT(gemm(300, 200, 250, 256, 256, 200), FP8MI_ERR_SHAPE);
  EXPECT(gemm(kMax, kMax, kMax, kMax, kMax, kMax), FP8MI_ERR_SHAPE);
  EXPECT(gemm(kMax, kMax, 0, 0, 0, kMax), FP8MI_ERR_SHAPE);
  EXPECT(gemm(1LL << 31, 16, 16, 16, 16, kMax), FP8MI_ERR_SHAPE);
  EXPECT(gemm(0x7FFFFFFF, 16, 16, 16, 16, 1LL << 40, FP8MI_GEMM_TENSOR, P, FP8MI_OUT_FP32), FP8MI_ERR_SHAPE);
  EXPECT(gemm(kMin, 16, 16, 16, 16, 16), FP8MI_ERR_SHAPE);
  EXPECT(fp8_bf16_gemm(P, kMax, P, kMax, kMax, kMax, kMax, P, FP8MI_OUT_BF16, kMax, nullptr), FP8MI_ERR_SHAPE);
  EXPECT(fp8_bf16_gemm(P, 64, P, 64, 1LL << 30, 64, 64, P, FP8MI_OUT_FP32, 1LL << 40, nullptr), FP8MI_ERR_SHAPE);
  EXPECT(fp8_bf16_gemm(P, 64, P, 64, 128, 64, 64, P, FP8MI_OUT_BF16, 64, nullptr), FP8MI_OK);

  // ---- status strings and version
  for (int s = -10; s <= 1; ++s)
    if (!fp8_status_string(s)) EXPECT(0, 1);
  EXPECT((int)(fp8_version() > 0), 1);

  if (g_failures) {
    printf("%d failure(s)\n", g_failures);
    return 1;
  }
  printf("abi validation ok\n");
  return 0;
}
