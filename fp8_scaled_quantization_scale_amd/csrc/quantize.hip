// quantize.hip -- scaled FP8 quantization kernels for gfx950.
//
// Recipes ("2025 technical guide: FP8 quantized training"):
//   sec. 2.1  per-tensor current scaling (amax of the tensor now) and delayed
//             scaling (scale carried over from the amax history);
//   sec. 2.2  blockwise: 1x128 tiles for activations / gradients, 128x128
//             tiles for weights, one scale per tile;
//   sec. 2.3  MXFP8: 1x32 blocks with E8M0 power-of-two scales.
// "Mastering FP8 LLM training", strategy 3: finer blocks must be
// re-quantized when the operand is used transposed -- the COL layout below
// (wgrad operands run their blocks along the token dimension M).
//
// One kernel handles every recipe and orientation on 128 x 128 tiles:
//   * each workgroup (256 threads) reads one tile once with 16-byte loads; a
//     16-lane group owns one tile row per step (16 lanes x 8 elements);
//   * ROW codes/scales are produced from registers: 1x128 blocks reduce over
//     the 16 lanes of a group, MX 1x32 blocks over 4 lanes, 128x128 tiles
//     over the workgroup;
//   * COL codes are the transposed layout: the tile is staged in LDS, each
//     thread walks half a column (64 rows), and the codes of 64 consecutive
//     rows leave as 64 contiguous bytes of the transposed output row.
// Per-tensor current scaling needs the amax of the whole tensor before any
// cast, so it runs a separate reduction kernel first.
#include "device.hpp"
#include "launch.hpp"

namespace fp8mi {

namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

enum : int { MODE_TENSOR = 0, MODE_B1x128 = 1, MODE_B128x128 = 2, MODE_MX32 = 3 };

template <typename InT>
struct In;
template <>
struct In<uint16_t> {  // BF16 bits
  static __device__ __forceinline__ float to_f(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
  }
  static __device__ __forceinline__ uint16_t from_f(float f) {
    return (uint16_t)(__builtin_bit_cast(uint32_t, f) >> 16);
  }
};
template <>
struct In<float> {
  static __device__ __forceinline__ float to_f(float h) { return h; }
  static __device__ __forceinline__ float from_f(float f) { return f; }
};

// 8 consecutive elements starting at p, `n` of them valid (zero beyond).
__device__ __forceinline__ void load8(const uint16_t* p, int64_t n, float v[8]) {
  if (n >= 8) {
    uint4 w = *reinterpret_cast<const uint4*>(p);
    unpack_bf16x8(w, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < n ? In<uint16_t>::to_f(p[e]) : 0.0f;
  }
}
__device__ __forceinline__ void load8(const float* p, int64_t n, float v[8]) {
  if (n >= 8) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < n ? p[e] : 0.0f;
  }
}

template <int FMT, bool Safe>
__device__ __forceinline__ uint2 encode8(const float v[8], float s) {
  uint2 r;
  r.x = encode4<FMT, Safe>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
  r.y = encode4<FMT, Safe>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
  return r;
}

__device__ __forceinline__ void store8(uint8_t* q, int64_t n, uint2 c) {
  if (n >= 8) {
    *reinterpret_cast<uint2*>(q) = c;
  } else {
    for (int e = 0; e < n; ++e) q[e] = (uint8_t)((e < 4 ? c.x >> (8 * e) : c.y >> (8 * (e - 4))) & 0xFF);
  }
}

__device__ __forceinline__ uint32_t max8_key(const float v[8]) {
  uint32_t k = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t t = abs_key(v[e]);
    k = k > t ? k : t;
  }
  return k;
}

// Workgroup-wide unsigned max; every thread gets the result.
__device__ __forceinline__ uint32_t wg_max_u32(uint32_t v, uint32_t* red4) {
  v = group_max_u32<64>(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red4 may still be read by an earlier reduction
  if ((threadIdx.x & 63) == 0) red4[wave] = v;
  __syncthreads();
  uint32_t a = red4[0] > red4[1] ? red4[0] : red4[1];
  uint32_t b = red4[2] > red4[3] ? red4[2] : red4[3];
  return a > b ? a : b;
}

struct TileArgs {
  const void* x;
  int64_t rows, cols, ld_x;
  uint8_t* q_row;
  int64_t ld_q_row;
  void* s_row;
  uint8_t* q_col;
  int64_t ld_q_col;
  void* s_col;
  float* scale;       // per-tensor: in (delayed) / out (current)
  float* scale_inv;   // per-tensor current: out
  float* amax;        // per-tensor: in (current) / max-accumulated (delayed)
  int32_t* nonfinite;
  int margin;
};

// CURRENT: per-tensor scale from the finished amax; DELAYED: given scale.
template <typename InT, int FMT, int MODE, bool ROW, bool COL, bool CURRENT>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(TileArgs a) {
  constexpr int kLdsElems = COL ? kTile * kTile : 1;
  __shared__ InT tile[kLdsElems];
  __shared__ uint32_t red4[4];
  __shared__ uint32_t colred[2][kTile];

  const int tid = threadIdx.x;
  const int g = tid >> 4;   // row group 0..15
  const int li = tid & 15;  // lane in group
  const int64_t row0 = (int64_t)blockIdx.y * kTile;
  const int64_t col0 = (int64_t)blockIdx.x * kTile;
  const int64_t ccol = col0 + 8 * li;  // first column of this lane's chunk
  const int64_t nval = a.cols - ccol;  // valid elements in the chunk (may be <= 0)
  const InT* x = reinterpret_cast<const InT*>(a.x);

  // ---- load the tile: rows g, g+16, ..., g+112
  float v[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + g + 16 * i;
    if (r < a.rows && nval > 0) {
      load8(x + r * a.ld_x + ccol, nval, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
    }
  }

  // ---- per-tensor and per-tile scales
  float s_t = 1.0f;
  bool safe_t = true;
  if constexpr (MODE == MODE_TENSOR) {
    if constexpr (CURRENT) {
      const float am = *a.amax;
      s_t = scale_from_amax<FMT>(am, a.margin);
      safe_t = !is_finite(am);
      if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
        *a.scale = s_t;
        *a.scale_inv = recip_rn(s_t);
        if (safe_t && a.nonfinite) atomicAdd(a.nonfinite, 1);
      }
    } else {
      s_t = *a.scale;
      uint32_t k = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t t = max8_key(v[i]);
        k = k > t ? k : t;
      }
      k = wg_max_u32(k, red4);
      if (tid == 0) atomicMax(reinterpret_cast<uint32_t*>(a.amax), k);
    }
  } else if constexpr (MODE == MODE_B128x128) {
    uint32_t k = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t t = max8_key(v[i]);
      k = k > t ? k : t;
    }
    k = wg_max_u32(k, red4);
    const float am = key_to_float(k);
    s_t = scale_from_amax<FMT>(am, a.margin);
    safe_t = !is_finite(am);
    if (tid == 0) {
      const float si = recip_rn(s_t);
      const int64_t gr = (a.rows + kTile - 1) / kTile, gc = (a.cols + kTile - 1) / kTile;
      if (ROW) reinterpret_cast<float*>(a.s_row)[blockIdx.y * gc + blockIdx.x] = si;
      if (COL) reinterpret_cast<float*>(a.s_col)[blockIdx.x * gr + blockIdx.y] = si;
      if (safe_t && a.nonfinite) atomicAdd(a.nonfinite, 1);
    }
  }

  // ---- ROW layout, straight from registers
  if constexpr (ROW) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = row0 + g + 16 * i;
      float s = s_t;
      bool safe = safe_t;
      if constexpr (MODE == MODE_B1x128) {
        const uint32_t k = group_max_u32<16>(max8_key(v[i]));
        const float am = key_to_float(k);
        s = scale_from_amax<FMT>(am, a.margin);
        safe = !is_finite(am);
        if (li == 0 && r < a.rows) {
          const int64_t gc = (a.cols + kTile - 1) / kTile;
          reinterpret_cast<float*>(a.s_row)[r * gc + blockIdx.x] = recip_rn(s);
          if (safe && a.nonfinite) atomicAdd(a.nonfinite, 1);
        }
      } else if constexpr (MODE == MODE_MX32) {
        const uint32_t k = group_max_u32<4>(max8_key(v[i]));
        const int byte = mx_scale_byte<FMT>(key_to_float(k));
        safe = byte == 0xFF;
        s = safe ? 1.0f : mx_inv_scale(byte);
        if ((li & 3) == 0 && r < a.rows && nval > 0) {
          const int64_t gc = (a.cols + 31) / 32;
          reinterpret_cast<uint8_t*>(a.s_row)[r * gc + (ccol >> 5)] = (uint8_t)byte;
          if (safe && a.nonfinite) atomicAdd(a.nonfinite, 1);
        }
      } else if constexpr (MODE == MODE_TENSOR && !CURRENT) {
        safe = true;
      }
      if (r < a.rows && nval > 0) {
        uint2 c = safe ? encode8<FMT, true>(v[i], s) : encode8<FMT, false>(v[i], s);
        store8(a.q_row + r * a.ld_q_row + ccol, nval, c);
      }
    }
  }

  // ---- COL layout: transpose through LDS
  if constexpr (COL) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = g + 16 * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rl * kTile + 8 * li + e] = In<InT>::from_f(v[i][e]);
    }
    __syncthreads();

    const int c = tid & (kTile - 1);  // tile column
    const int h = tid >> 7;           // rows 64h .. 64h+63
    const int64_t col = col0 + c;
    const int64_t rbase = row0 + 64 * h;
    float w[64];
#pragma unroll
    for (int j = 0; j < 64; ++j) w[j] = In<InT>::to_f(tile[(64 * h + j) * kTile + c]);

    float s0 = s_t, s1 = s_t;  // scales for rows [0,32) and [32,64) of this half
    bool safe0 = safe_t, safe1 = safe_t;
    if constexpr (MODE == MODE_TENSOR && !CURRENT) {
      safe0 = safe1 = true;
    } else if constexpr (MODE == MODE_B1x128) {
      uint32_t k = 0;
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        uint32_t t = abs_key(w[j]);
        k = k > t ? k : t;
      }
      colred[h][c] = k;
      __syncthreads();
      k = colred[0][c] > colred[1][c] ? colred[0][c] : colred[1][c];
      const float am = key_to_float(k);
      s0 = s1 = scale_from_amax<FMT>(am, a.margin);
      safe0 = safe1 = !is_finite(am);
      if (h == 0 && col < a.cols) {
        const int64_t gr = (a.rows + kTile - 1) / kTile;
        reinterpret_cast<float*>(a.s_col)[col * gr + blockIdx.y] = recip_rn(s0);
        if (safe0 && a.nonfinite) atomicAdd(a.nonfinite, 1);
      }
    } else if constexpr (MODE == MODE_MX32) {
      uint32_t k0 = 0, k1 = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        uint32_t t0 = abs_key(w[j]), t1 = abs_key(w[32 + j]);
        k0 = k0 > t0 ? k0 : t0;
        k1 = k1 > t1 ? k1 : t1;
      }
      const int b0 = mx_scale_byte<FMT>(key_to_float(k0));
      const int b1 = mx_scale_byte<FMT>(key_to_float(k1));
      safe0 = b0 == 0xFF;
      safe1 = b1 == 0xFF;
      s0 = safe0 ? 1.0f : mx_inv_scale(b0);
      s1 = safe1 ? 1.0f : mx_inv_scale(b1);
      if (col < a.cols) {
        const int64_t gr = (a.rows + 31) / 32;
        uint8_t* sc = reinterpret_cast<uint8_t*>(a.s_col) + col * gr;
        if (rbase < a.rows) {
          sc[rbase >> 5] = (uint8_t)b0;
          if (safe0 && a.nonfinite) atomicAdd(a.nonfinite, 1);
        }
        if (rbase + 32 < a.rows) {
          sc[(rbase >> 5) + 1] = (uint8_t)b1;
          if (safe1 && a.nonfinite) atomicAdd(a.nonfinite, 1);
        }
      }
    }

    if (col < a.cols && rbase < a.rows) {
      uint32_t pk[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float s = q < 8 ? s0 : s1;
        const bool safe = q < 8 ? safe0 : safe1;
        pk[q] = safe ? encode4<FMT, true>(w[4 * q] * s, w[4 * q + 1] * s, w[4 * q + 2] * s, w[4 * q + 3] * s)
                     : encode4<FMT, false>(w[4 * q] * s, w[4 * q + 1] * s, w[4 * q + 2] * s, w[4 * q + 3] * s);
      }
      uint8_t* dst = a.q_col + col * a.ld_q_col + rbase;
      const int64_t n = a.rows - rbase;
      if (n >= 64) {
        uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
        for (int q = 0; q < 4; ++q) d4[q] = make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
      } else {
        for (int j = 0; j < n; ++j) dst[j] = (uint8_t)((pk[j >> 2] >> (8 * (j & 3))) & 0xFF);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-tensor amax for current scaling: max |x| over the tensor, NaN-dominant,
// max-accumulated into *amax (zeroed by zero_kernel first).
// ---------------------------------------------------------------------------
__global__ void zero_kernel(float* p) { *p = 0.0f; }

template <typename InT>
__global__ __launch_bounds__(kThreads) void amax_kernel(const InT* x, int64_t rows, int64_t cols,
                                                        int64_t ld, float* amax) {
  __shared__ uint32_t red4[4];
  const int64_t cpr = (cols + 7) / 8;
  const int64_t total = rows * cpr;
  uint32_t k = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / cpr;
    const int64_t cc = (i - r * cpr) * 8;
    float v[8];
    load8(x + r * ld + cc, cols - cc, v);
    const uint32_t t = max8_key(v);
    k = k > t ? k : t;
  }
  k = wg_max_u32(k, red4);
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<uint32_t*>(amax), k);
}

template <typename InT, int FMT, int MODE, bool CURRENT>
hipError_t launch_tile(const QuantParams& p, hipStream_t st) {
  TileArgs a{p.x, p.rows, p.cols, p.ld_x, p.q_row, p.ld_q_row, p.s_row, p.q_col, p.ld_q_col,
             p.s_col, p.scale, p.scale_inv, p.amax, p.nonfinite, p.margin};
  dim3 grid((unsigned)((p.cols + kTile - 1) / kTile), (unsigned)((p.rows + kTile - 1) / kTile));
  const bool row = p.orient & 1, col = p.orient & 2;
  if (row && col)
    quant_tile_kernel<InT, FMT, MODE, true, true, CURRENT><<<grid, kThreads, 0, st>>>(a);
  else if (row)
    quant_tile_kernel<InT, FMT, MODE, true, false, CURRENT><<<grid, kThreads, 0, st>>>(a);
  else
    quant_tile_kernel<InT, FMT, MODE, false, true, CURRENT><<<grid, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <typename InT, int FMT>
hipError_t launch_fmt(const QuantParams& p, hipStream_t st) {
  switch (p.recipe) {
    case kRecipeTensorCurrent: {
      zero_kernel<<<1, 1, 0, st>>>(p.amax);
      if (p.rows > 0 && p.cols > 0) {
        const int64_t chunks = p.rows * ((p.cols + 7) / 8);
        int64_t blocks = (chunks + kThreads - 1) / kThreads;
        blocks = blocks < 2048 ? blocks : 2048;
        amax_kernel<InT><<<(unsigned)blocks, kThreads, 0, st>>>(
            reinterpret_cast<const InT*>(p.x), p.rows, p.cols, p.ld_x, p.amax);
        return launch_tile<InT, FMT, MODE_TENSOR, true>(p, st);
      }
      // empty tensor: amax = 0 -> scale = scale_inv = 1
      return launch_empty_scale(p.scale, p.scale_inv, st);
    }
    case kRecipeTensorDelayed:
      if (p.rows == 0 || p.cols == 0) return hipGetLastError();
      return launch_tile<InT, FMT, MODE_TENSOR, false>(p, st);
    case kRecipeBlock1x128:
      return launch_tile<InT, FMT, MODE_B1x128, false>(p, st);
    case kRecipeBlock128x128:
      return launch_tile<InT, FMT, MODE_B128x128, false>(p, st);
    case kRecipeMx1x32:
      return launch_tile<InT, FMT, MODE_MX32, false>(p, st);
  }
  return hipErrorInvalidValue;
}

__global__ void empty_scale_kernel(float* scale, float* scale_inv) {
  *scale = 1.0f;
  *scale_inv = 1.0f;
}

}  // namespace

hipError_t launch_empty_scale(float* scale, float* scale_inv, hipStream_t st) {
  empty_scale_kernel<<<1, 1, 0, st>>>(scale, scale_inv);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t st) {
  if (p.recipe != kRecipeTensorCurrent && (p.rows == 0 || p.cols == 0)) return hipSuccess;
  if (p.x_dtype == kInBf16) {
    return p.fmt == kE4M3 ? launch_fmt<uint16_t, kE4M3>(p, st) : launch_fmt<uint16_t, kE5M2>(p, st);
  }
  return p.fmt == kE4M3 ? launch_fmt<float, kE4M3>(p, st) : launch_fmt<float, kE5M2>(p, st);
}

}  // namespace fp8mi
