// probe.hip -- measurement kernels behind include/fp8mi_probe.h: the matrix
// cores' rate and the shader clock under full FP8 MFMA load, and plain HBM
// streams at the quantize kernels' read:write mixes.  They bound what the
// FP8 path can reach on this GPU; they are not part of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8mi_probe.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kMfmaWaves = 8;  // two waves per SIMD
constexpr int kMfmaAcc = 8;    // independent products in flight per wave

__device__ __forceinline__ uint4 xor4(uint4 a, uint4 b) { return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w); }

// Every access is at an index below its bound (n for src, n or n / 2 for
// dst0 / dst1): the loop conditions check the largest index of each trip.
template <int MIX>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const uint4* __restrict__ src, int64_t n,
                                                                uint4* __restrict__ dst0, uint4* __restrict__ dst1) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  if constexpr (MIX == FP8PROBE_READ || MIX == FP8PROBE_COPY) {
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (; i + 3 * stride < n; i += 4 * stride) {
      const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
      if constexpr (MIX == FP8PROBE_COPY) {
        dst0[i] = a;
        dst0[i + stride] = b;
        dst0[i + 2 * stride] = c;
        dst0[i + 3 * stride] = d;
      } else {
        acc = xor4(acc, xor4(xor4(a, b), xor4(c, d)));
      }
    }
    for (; i < n; i += stride) {
      const uint4 a = src[i];
      if constexpr (MIX == FP8PROBE_COPY) dst0[i] = a;
      else acc = xor4(acc, a);
    }
    if constexpr (MIX == FP8PROBE_READ) {
      if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0xF39CC060u && acc.w == 0x5CEDC834u) dst0[0] = acc;
    }
  } else {
    const int64_t h = n / 2;  // output chunks
    for (; i + 3 * stride < h; i += 4 * stride) {
      uint4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = src[2 * (i + u * stride)];
        b[u] = src[2 * (i + u * stride) + 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (MIX == FP8PROBE_HALF) {
          dst0[i + u * stride] = xor4(a[u], b[u]);
        } else {
          dst0[i + u * stride] = a[u];
          dst1[i + u * stride] = b[u];
        }
      }
    }
    for (; i < h; i += stride) {
      const uint4 a = src[2 * i], b = src[2 * i + 1];
      if constexpr (MIX == FP8PROBE_HALF) {
        dst0[i] = xor4(a, b);
      } else {
        dst0[i] = a;
        dst1[i] = b;
      }
    }
  }
}

__global__ __launch_bounds__(64 * kMfmaWaves) void mfma_kernel(int iters, uint64_t* clocks, float* sink) {
  v8i a, b;  // E4M3 codes of 1.0 and 0.5, perturbed per lane
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ (t & 7);
    b[i] = 0x30303030 ^ ((t >> 3) & 7);
  }
  v4f acc[kMfmaAcc];
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();
  const uint64_t c0 = (uint64_t)clock64(), w0 = (uint64_t)wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
  }
  __syncthreads();
  const uint64_t c1 = (uint64_t)clock64(), w1 = (uint64_t)wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 1234.5678f) sink[0] = s;
  if (t == 0) {
    clocks[4 * blockIdx.x + 0] = c0;
    clocks[4 * blockIdx.x + 1] = c1;
    clocks[4 * blockIdx.x + 2] = w0;
    clocks[4 * blockIdx.x + 3] = w1;
  }
}

int stream_device(hipStream_t st) {
  int dev = -1;
  if (st == nullptr || hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0)
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return dev;
}

int device_cus(hipStream_t st) {
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, stream_device(st)) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -6; }

}  // namespace

extern "C" {

int fp8probe_stream(const void* src, int64_t n16, void* dst0, void* dst1, int mix, void* stream) {
  if (mix < FP8PROBE_READ || mix > FP8PROBE_SPLIT) return -2;
  if (n16 < 0 || ((mix == FP8PROBE_HALF || mix == FP8PROBE_SPLIT) && (n16 & 1))) return -3;
  if (!src || !dst0 || (mix == FP8PROBE_SPLIT && !dst1)) return -1;
  if (((uintptr_t)src | (uintptr_t)dst0 | (uintptr_t)dst1) & 15u) return -5;
  if (n16 == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const int64_t work = (mix == FP8PROBE_HALF || mix == FP8PROBE_SPLIT) ? n16 / 2 : n16;
  int64_t blocks = (int64_t)device_cus(st) * 8;
  const int64_t need = (work + kStreamThreads - 1) / kStreamThreads;
  blocks = blocks < need ? blocks : need;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d0 = reinterpret_cast<uint4*>(dst0);
  uint4* d1 = reinterpret_cast<uint4*>(dst1);
  switch (mix) {
    case FP8PROBE_READ: stream_kernel<FP8PROBE_READ><<<(unsigned)blocks, kStreamThreads, 0, st>>>(s, n16, d0, d1); break;
    case FP8PROBE_COPY: stream_kernel<FP8PROBE_COPY><<<(unsigned)blocks, kStreamThreads, 0, st>>>(s, n16, d0, d1); break;
    case FP8PROBE_HALF: stream_kernel<FP8PROBE_HALF><<<(unsigned)blocks, kStreamThreads, 0, st>>>(s, n16, d0, d1); break;
    default: stream_kernel<FP8PROBE_SPLIT><<<(unsigned)blocks, kStreamThreads, 0, st>>>(s, n16, d0, d1); break;
  }
  return launched();
}

int fp8probe_mfma(int iters, int workgroups, uint64_t* clocks, float* sink, void* stream) {
  if (iters < 1 || workgroups < 1) return -3;
  if (!clocks || !sink) return -1;
  mfma_kernel<<<(unsigned)workgroups, 64 * kMfmaWaves, 0, (hipStream_t)stream>>>(iters, clocks, sink);
  return launched();
}

int fp8probe_wall_clock_khz(void* stream) {
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, stream_device((hipStream_t)stream)) != hipSuccess ||
      khz <= 0)
    return -6;
  return khz;
}

}  // extern "C"
