// probe.hip -- measurement kernels behind include/fp8mi_probe.h: the matrix
// cores' rate and the shader clock under full FP8 MFMA load (fixed or varied
// operands), and plain HBM
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

constexpr int kMfmaLdsWords = 96 * 1024 / 4;  // one workgroup per compute unit

__device__ __forceinline__ uint4 xor4(uint4 a, uint4 b) { return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld(const uint4* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}
template <bool NT>
__device__ __forceinline__ void st(uint4* p, uint4 v) {
  if constexpr (NT) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  } else {
    *p = v;
  }
}

// Work item i of a pass reads src[i] (READ, COPY) or src[2i], src[2i+1]
// (HALF, SPLIT) and writes its output chunk(s) at i; there are n items (READ,
// COPY) or n / 2.  Grid-strided: thread t of workgroup b takes items
// b * 256 + t + k * (grid * 256).  BLOCKED: workgroup b takes the contiguous
// range [b * per, (b + 1) * per) of items, thread t every 256th of it.
// Eight 16-byte loads are in flight per thread per trip.  Every access is at
// an index below its bound (n for src, n or n / 2 for dst0 / dst1): each
// trip's largest item index is checked against the item count.
template <int MIX, bool NTL, bool NTS, bool BLOCKED>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const uint4* __restrict__ src, int64_t n,
                                                                uint4* __restrict__ dst0, uint4* __restrict__ dst1) {
  constexpr bool kPair = MIX == FP8PROBE_HALF || MIX == FP8PROBE_SPLIT;
  constexpr int U = kPair ? 4 : 8;  // items per trip (8 loads either way)
  const int64_t items = kPair ? n / 2 : n;
  int64_t i, end, step;
  if constexpr (BLOCKED) {
    const int64_t per = (items + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    end = b0 + per < items ? b0 + per : items;
    i = b0 + threadIdx.x;
    step = kStreamThreads;
  } else {
    end = items;
    i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    step = (int64_t)gridDim.x * kStreamThreads;
  }
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (; i + (U - 1) * step < end; i += U * step) {
    uint4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (kPair) {
        a[u] = ld<NTL>(src + 2 * (i + u * step));
        b[u] = ld<NTL>(src + 2 * (i + u * step) + 1);
      } else {
        a[u] = ld<NTL>(src + i + u * step);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (MIX == FP8PROBE_READ) acc = xor4(acc, a[u]);
      else if constexpr (MIX == FP8PROBE_COPY) st<NTS>(dst0 + i + u * step, a[u]);
      else if constexpr (MIX == FP8PROBE_HALF) st<NTS>(dst0 + i + u * step, xor4(a[u], b[u]));
      else {
        st<NTS>(dst0 + i + u * step, a[u]);
        st<NTS>(dst1 + i + u * step, b[u]);
      }
    }
  }
  for (; i < end; i += step) {
    if constexpr (kPair) {
      const uint4 a = ld<NTL>(src + 2 * i), b = ld<NTL>(src + 2 * i + 1);
      if constexpr (MIX == FP8PROBE_HALF) {
        st<NTS>(dst0 + i, xor4(a, b));
      } else {
        st<NTS>(dst0 + i, a);
        st<NTS>(dst1 + i, b);
      }
    } else {
      const uint4 a = ld<NTL>(src + i);
      if constexpr (MIX == FP8PROBE_READ) acc = xor4(acc, a);
      else st<NTS>(dst0 + i, a);
    }
  }
  if constexpr (MIX == FP8PROBE_READ) {
    if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0xF39CC060u && acc.w == 0x5CEDC834u) dst0[0] = acc;
  }
}

// Per-lane hash (a 32-bit integer mixer) for the varied operands.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// SETS == 1: every product multiplies the same codes (E4M3 1.0 and 0.5,
// perturbed per lane), so the multipliers barely switch and the clock is
// the chip's limit.  SETS == 4: four operand sets per lane from the hash
// (E4M3 codes with the lowest exponent bit cleared, which excludes the NaN
// pattern), cycled so that each product multiplies other codes than the one
// before it, as in a GEMM.
template <int SETS>
__global__ __launch_bounds__(64 * kMfmaWaves) void mfma_kernel(int iters, uint64_t* clocks, float* sink) {
  __shared__ float pad[kMfmaLdsWords];  // holds the compute unit: one workgroup each
  v8i a[SETS], b[SETS];
  const int t = threadIdx.x;
#pragma unroll
  for (int s = 0; s < SETS; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (SETS == 1) {
        a[s][i] = 0x38383838 ^ (t & 7);
        b[s][i] = 0x30303030 ^ ((t >> 3) & 7);
      } else {
        const uint32_t h = ((blockIdx.x * 64u * kMfmaWaves + (uint32_t)t) * SETS + (uint32_t)s) * 8u + (uint32_t)i;
        a[s][i] = (int)(mix32(h) & 0xF7F7F7F7u);
        b[s][i] = (int)(mix32(h ^ 0x9E3779B9u) & 0xF7F7F7F7u);
      }
    }
  v4f acc[kMfmaAcc];
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();
  const uint64_t c0 = (uint64_t)clock64(), w0 = (uint64_t)wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j % SETS], b[(j + j / SETS) % SETS], acc[j], 0, 0, 0,
                                                                 0, 0, 0);
  }
  __syncthreads();
  const uint64_t c1 = (uint64_t)clock64(), w1 = (uint64_t)wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  pad[t] = s;
  __syncthreads();
  if (pad[(t + 1) % (64 * kMfmaWaves)] == 1234.5678f) sink[0] = s;
  if (t == 0) {
    clocks[4 * blockIdx.x + 0] = c0;
    clocks[4 * blockIdx.x + 1] = c1;
    clocks[4 * blockIdx.x + 2] = w0;
    clocks[4 * blockIdx.x + 3] = w1;
  }
}

// Does nothing: a dispatch of it costs what any launch of that shape costs.
__global__ void empty_kernel() {}

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
  if ((mix & ~(15 | FP8PROBE_NT_LOAD | FP8PROBE_NT_STORE | FP8PROBE_BLOCKED)) || (mix & 15) > FP8PROBE_SPLIT) return -2;
  const int base = mix & 15;
  if (n16 < 0 || ((base == FP8PROBE_HALF || base == FP8PROBE_SPLIT) && (n16 & 1))) return -3;
  if (!src || !dst0 || (base == FP8PROBE_SPLIT && !dst1)) return -1;
  if (((uintptr_t)src | (uintptr_t)dst0 | (uintptr_t)dst1) & 15u) return -5;
  if (n16 == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const int64_t work = (base == FP8PROBE_HALF || base == FP8PROBE_SPLIT) ? n16 / 2 : n16;
  int64_t blocks = (int64_t)device_cus(st) * 8;
  const int64_t need = (work + kStreamThreads - 1) / kStreamThreads;
  blocks = blocks < need ? blocks : need;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d0 = reinterpret_cast<uint4*>(dst0);
  uint4* d1 = reinterpret_cast<uint4*>(dst1);
  const bool ntl = (mix & FP8PROBE_NT_LOAD) != 0, nts = (mix & FP8PROBE_NT_STORE) != 0;
  const bool blk = (mix & FP8PROBE_BLOCKED) != 0;
  auto go = [&](auto k) { k<<<(unsigned)blocks, kStreamThreads, 0, st>>>(s, n16, d0, d1); };
#define FP8PROBE_LAUNCH2(M, B)                                    \
  if (ntl && nts) go(stream_kernel<M, true, true, B>);            \
  else if (ntl) go(stream_kernel<M, true, false, B>);             \
  else if (nts) go(stream_kernel<M, false, true, B>);             \
  else go(stream_kernel<M, false, false, B>);
#define FP8PROBE_LAUNCH(M) \
  if (blk) { FP8PROBE_LAUNCH2(M, true) } else { FP8PROBE_LAUNCH2(M, false) }
  switch (base) {
    case FP8PROBE_READ: FP8PROBE_LAUNCH(FP8PROBE_READ) break;
    case FP8PROBE_COPY: FP8PROBE_LAUNCH(FP8PROBE_COPY) break;
    case FP8PROBE_HALF: FP8PROBE_LAUNCH(FP8PROBE_HALF) break;
    default: FP8PROBE_LAUNCH(FP8PROBE_SPLIT) break;
  }
#undef FP8PROBE_LAUNCH2
#undef FP8PROBE_LAUNCH
  return launched();
}

int fp8probe_mfma(int iters, int workgroups, uint64_t* clocks, float* sink, void* stream) {
  if (iters < 1 || workgroups < 1) return -3;
  if (!clocks || !sink) return -1;
  mfma_kernel<1><<<(unsigned)workgroups, 64 * kMfmaWaves, 0, (hipStream_t)stream>>>(iters, clocks, sink);
  return launched();
}

int fp8probe_mfma_varied(int iters, int workgroups, uint64_t* clocks, float* sink, void* stream) {
  if (iters < 1 || workgroups < 1) return -3;
  if (!clocks || !sink) return -1;
  mfma_kernel<4><<<(unsigned)workgroups, 64 * kMfmaWaves, 0, (hipStream_t)stream>>>(iters, clocks, sink);
  return launched();
}

int fp8probe_empty(int workgroups, int threads, void* stream) {
  if (workgroups < 1 || threads < 1 || threads > 1024) return -3;
  empty_kernel<<<(unsigned)workgroups, (unsigned)threads, 0, (hipStream_t)stream>>>();
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
