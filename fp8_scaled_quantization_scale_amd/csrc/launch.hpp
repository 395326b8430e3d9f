// launch.hpp -- internal launchers behind the C ABI (include/fp8mi.h).
// Arguments arrive here already validated by the host-side checks in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fp8mi {

// ---- the device a launch runs on, and its size -------------------------
// Work goes to the caller's stream, whose device need not be the current
// one; persistent grids are sized for that device (a partitioned GPU
// exposes devices with fewer compute units).
constexpr int kMaxDevices = 64;

inline int stream_device(hipStream_t st) {
  int dev = -1;
  if (st != nullptr && hipStreamGetDevice(st, &dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) return dev;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  return dev;
}

// Compute units of device `dev`, queried once per process and device.  The
// cache is atomic: concurrent first calls store the same value.
inline int cu_count(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// values mirror the FP8MI_* macros of the public header
constexpr int kInBf16 = 0, kInFp32 = 1;
constexpr int kOutBf16 = 0, kOutFp32 = 1;
constexpr int kRecipeTensorCurrent = 0, kRecipeTensorDelayed = 1, kRecipeBlock1x128 = 2,
              kRecipeBlock128x128 = 3, kRecipeMx1x32 = 4, kRecipeChannel = 5, kRecipeMx1x32Ocp = 6;
constexpr int kGemmTensor = 0, kGemmBlock128x128 = 1, kGemmBlock1x128 = 2, kGemmMx = 3, kGemmBlock2d = 4,
              kGemmChannel = 5;
// internal: BF16 operands, no scales (fp8_bf16_gemm)
constexpr int kGemmBf16 = 16;
// slots of a delayed-scaling amax accumulator (FP8MI_AMAX_SLOTS)
constexpr int kAmaxSlots = 1024;

struct QuantParams {
  const void* x;
  int x_dtype;
  int64_t rows, cols, ld_x;
  int recipe, fmt, orient, margin;
  uint8_t* q_row;
  int64_t ld_q_row;
  void* s_row;
  uint8_t* q_col;
  int64_t ld_q_col;
  void* s_col;
  float* scale;
  float* scale_inv;
  float* amax;
  int32_t* nonfinite;
  // current scaling: where the amax pass leaves its per-workgroup partial
  // maxima (nullptr: amax[1 ..], the caller's array)
  uint32_t* partials = nullptr;
};

struct GemmParams {
  const uint8_t* a;
  int fmt_a;
  const void* s_a;
  int64_t lda;
  const uint8_t* b;
  int fmt_b;
  const void* s_b;
  int64_t ldb;
  int recipe;
  int64_t M, N, K;
  void* c;
  int c_dtype;
  int64_t ldc;
};

hipError_t launch_quantize(const QuantParams& p, hipStream_t st);
// fp8_quantize with current scaling's partial maxima in the library's static
// device scratch instead of amax[1 ..] (see quantize.hip)
hipError_t launch_quantize_static_scratch(const QuantParams& p, hipStream_t st);
hipError_t launch_empty_scale(float* amax, float* scale, float* scale_inv, hipStream_t st);
hipError_t launch_history(float* history, int32_t* head, int len, float* amax, int fmt, int margin,
                          float* scale, float* scale_inv, int32_t* nonfinite, hipStream_t st);
hipError_t launch_gemm(const GemmParams& p, hipStream_t st);
// a, b BF16 [M x K], [N x K]; K, lda, ldb in elements
hipError_t launch_gemm_bf16(const GemmParams& p, hipStream_t st);

}  // namespace fp8mi
