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
//   * persistent workgroups (256 threads) walk the tiles, each read once with
//     16-byte loads while the previous tile is processed; a 16-lane group owns
//     one tile row per step (16 lanes x 8 elements);
//   * ROW codes/scales are produced from registers: 1x128 blocks reduce over
//     the 16 lanes of a group, MX 1x32 blocks over 4 lanes, 128x128 tiles
//     over the workgroup;
//   * COL codes are the transposed layout: the tile is staged in LDS, each
//     thread walks a column pair for 32 rows, and the codes go back through
//     LDS so that each output row leaves as whole 128-byte lines.
// Per-tensor current scaling needs the amax of the whole tensor before any
// cast: a reduction pass leaves one partial maximum per workgroup in the
// caller's amax array, and every workgroup of the cast folds those few
// partials itself before its first tile (workgroup 0 stores the result in
// amax[0]), so no launch is spent on the fold.  No kernel
// combines results across workgroups with atomics: on MI355X atomics on one
// address serialise (about 14 ns each), which for a thousand workgroups
// costs as much as the whole cast.
#include <atomic>
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace fp8mi {

namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;
// partial maxima of current scaling's amax pass: one per workgroup, at most
// this many whatever the tensor's size (the pass grid-strides)
constexpr int kMaxPartials = kAmaxSlots - 1;
// byte stride of the transposed code tile staged in LDS: 144 = 128 + 16 keeps
// 16-byte alignment and spreads the column writes of a wave over the banks
constexpr int kCodeStride = 144;

// ROW codes are written whole-line by consecutive lanes and not read again
// by this pass, so they are stored non-temporally (measured on MI355X: an
// 8192x4096 ROW cast 20.9 -> 18.6 us).  Non-temporal loads of the input and
// non-temporal COL stores measured slower.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st_stream8(void* p, uint2 w) {
  const u32x2_t v = {w.x, w.y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

enum : int { MODE_TENSOR = 0, MODE_B1x128 = 1, MODE_B128x128 = 2, MODE_MX32 = 3, MODE_CHANNEL = 4, MODE_MX32F = 5 };

// E8M0 byte of an MX block: MODE_MX32 takes the smallest power of two under
// which no element saturates, MODE_MX32F the OCP specification's floor rule.
template <int MODE, int FMT>
__device__ __forceinline__ int mx_byte(float amax) {
  if constexpr (MODE == MODE_MX32F) return mx_scale_byte_floor<FMT>(amax);
  else return mx_scale_byte<FMT>(amax);
}
// Channel scales travel between the passes as the scale s itself, with the
// sign bit marking a row / column whose amax was not finite (s = 1 there).
__device__ __forceinline__ float chan_s(float v) { return __builtin_fabsf(v); }
__device__ __forceinline__ bool chan_bad(float v) { return __builtin_signbit(v) != 0; }

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
    st_stream8(q, c);
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
  float* amax;        // per-tensor: out amax[0] (current) / slot accumulator (delayed)
  int32_t* nonfinite;
  int margin;
  int nparts;         // current: partial maxima in parts[0 .. nparts - 1]
  const uint32_t* parts;
};

// max |x| key of 8 BF16 values packed in a uint4: packed 16-bit max of the
// sign-cleared halves (non-negative BF16 orders like its bits, NaN on top).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x8_key(uint4 w) {
  u16x2 m = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu));
  const uint32_t k = m.x > m.y ? m.x : m.y;
  return k << 16;
}

// A thread's share of one tile: rows g, g+16, ..., g+112, columns
// [8 li, 8 li + 8) of the tile, as raw 16-byte words (BF16: one per row,
// FP32: two).  Loads past the tensor's edge are zero.
template <typename InT>
struct Raw;
template <>
struct Raw<uint16_t> {
  uint4 w[8];
  __device__ __forceinline__ void row(int i, float v[8]) const { unpack_bf16x8(w[i], v); }
  __device__ __forceinline__ uint32_t key(int i, const float*) const { return bf16x8_key(w[i]); }
  __device__ __forceinline__ void load(const uint16_t* x, int64_t ld, int64_t rows, int64_t r0, int64_t ccol,
                                       int64_t nval) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + 16 * i;
      if (r < rows && nval >= 8) {
        w[i] = ld16(x + r * ld + ccol);
      } else {
        uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < rows)
          for (int e = 0; e < 8 && e < nval; ++e) h[e] = x[r * ld + ccol + e];
        w[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
    }
  }
};
template <>
struct Raw<float> {
  float4 w[16];
  __device__ __forceinline__ uint32_t key(int, const float* v) const { return max8_key(v); }
  __device__ __forceinline__ void row(int i, float v[8]) const {
    v[0] = w[2 * i].x; v[1] = w[2 * i].y; v[2] = w[2 * i].z; v[3] = w[2 * i].w;
    v[4] = w[2 * i + 1].x; v[5] = w[2 * i + 1].y; v[6] = w[2 * i + 1].z; v[7] = w[2 * i + 1].w;
  }
  __device__ __forceinline__ void load(const float* x, int64_t ld, int64_t rows, int64_t r0, int64_t ccol,
                                       int64_t nval) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + 16 * i;
      if (r < rows && nval >= 8) {
        const uint4 lo = ld16(x + r * ld + ccol), hi = ld16(x + r * ld + ccol + 4);
        w[2 * i] = make_float4(__builtin_bit_cast(float, lo.x), __builtin_bit_cast(float, lo.y),
                               __builtin_bit_cast(float, lo.z), __builtin_bit_cast(float, lo.w));
        w[2 * i + 1] = make_float4(__builtin_bit_cast(float, hi.x), __builtin_bit_cast(float, hi.y),
                                   __builtin_bit_cast(float, hi.z), __builtin_bit_cast(float, hi.w));
      } else {
        float h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < rows)
          for (int e = 0; e < 8 && e < nval; ++e) h[e] = x[r * ld + ccol + e];
        w[2 * i] = make_float4(h[0], h[1], h[2], h[3]);
        w[2 * i + 1] = make_float4(h[4], h[5], h[6], h[7]);
      }
    }
  }
};

// Delayed scaling: the convert-only encoder is exact for a chunk whose
// largest magnitude m is finite with fl32(m * s) <= max (every product then
// rounds to at most max); anything else takes the saturating encoder.
template <int FMT>
__device__ __forceinline__ bool fits(uint32_t key, float s) {
  const float m = key_to_float(key);
  return m <= kFltMax && m * s <= Fmt<FMT>::kMax;
}

// Persistent workgroups: each walks tiles blockIdx.x, blockIdx.x + gridDim.x,
// ... and prefetches the next tile's raw words into registers while the
// current one is processed, so every workgroup always has a tile in flight.
// CURRENT: per-tensor scale from the finished amax; otherwise the recipe's own.
template <typename InT, int FMT, int MODE, bool ROW, bool COL, bool CURRENT>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(TileArgs a) {
  constexpr int kLdsElems = COL ? kTile * kTile : 1;
  __shared__ InT tile[kLdsElems];
  __shared__ uint32_t red4[4];
  __shared__ uint32_t colred[4][kTile];

  const int tid = threadIdx.x;
  const int g = tid >> 4;   // row group 0..15
  const int li = tid & 15;  // lane in group
  const InT* x = reinterpret_cast<const InT*>(a.x);
  const int64_t tiles_x = (a.cols + kTile - 1) / kTile;
  const int64_t tiles = tiles_x * ((a.rows + kTile - 1) / kTile);

  // the first tile's words are in flight while the scale is worked out
  Raw<InT> cur, nxt;
  int64_t t = blockIdx.x;
  if (t < tiles) {
    const int64_t by = t / tiles_x, bx = t - by * tiles_x;
    cur.load(x, a.ld_x, a.rows, by * kTile + g, bx * kTile + 8 * li, a.cols - (bx * kTile + 8 * li));
  }

  // ---- per-tensor scale (the same for every tile)
  float s_tensor = 1.0f;
  bool safe_tensor = true;
  if constexpr (MODE == MODE_TENSOR) {
    if constexpr (CURRENT) {
      // every workgroup folds the amax pass's partial maxima (a few KB, from
      // L2); none of them writes the slots, so there is no ordering to keep
      const uint32_t* slots = a.parts;
      uint32_t k = 0;
      for (int i = tid; i < a.nparts; i += kThreads) k = k > slots[i] ? k : slots[i];
      const float am = key_to_float(wg_max_u32(k, red4));
      s_tensor = scale_from_amax<FMT>(am, a.margin);
      safe_tensor = !is_finite(am);
      if (blockIdx.x == 0 && tid == 0) {
        *a.amax = am;
        *a.scale = s_tensor;
        *a.scale_inv = recip_rn(s_tensor);
        if (safe_tensor && a.nonfinite) atomicAdd(a.nonfinite, 1);
      }
    } else {
      s_tensor = *a.scale;
    }
  }
  // delayed: this workgroup's running max |x|, seeded with its slot of the
  // accumulator (slot blockIdx.x belongs to this workgroup alone; the grid
  // never exceeds kAmaxSlots)
  uint32_t amax_acc = 0;
  if constexpr (MODE == MODE_TENSOR && !CURRENT) {
    if (tid == 0) amax_acc = reinterpret_cast<const uint32_t*>(a.amax)[blockIdx.x];
  }

  for (; t < tiles; t += gridDim.x) {
    const int64_t by = t / tiles_x, bx = t - by * tiles_x;
    const int64_t tn = t + gridDim.x;
    if (tn < tiles) {
      const int64_t byn = tn / tiles_x, bxn = tn - byn * tiles_x;
      nxt.load(x, a.ld_x, a.rows, byn * kTile + g, bxn * kTile + 8 * li, a.cols - (bxn * kTile + 8 * li));
    }
    const int64_t row0 = by * kTile, col0 = bx * kTile;
    const int64_t ccol = col0 + 8 * li;  // first column of this lane's chunk
    const int64_t nval = a.cols - ccol;  // valid elements in the chunk (may be <= 0)

    // ---- per-tile scale (128x128 recipe)
    float s_t = s_tensor;
    bool safe_t = safe_tensor;
    if constexpr (MODE == MODE_B128x128) {
      uint32_t k = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v[8];
        if constexpr (sizeof(InT) == 4) cur.row(i, v);
        const uint32_t m = cur.key(i, v);
        k = k > m ? k : m;
      }
      k = wg_max_u32(k, red4);
      const float am = key_to_float(k);
      s_t = scale_from_amax<FMT>(am, a.margin);
      safe_t = !is_finite(am);
      if (tid == 0) {
        const float si = recip_rn(s_t);
        const int64_t gr = (a.rows + kTile - 1) / kTile;
        if (ROW) reinterpret_cast<float*>(a.s_row)[by * tiles_x + bx] = si;
        if (COL) reinterpret_cast<float*>(a.s_col)[bx * gr + by] = si;
        if (safe_t && a.nonfinite) atomicAdd(a.nonfinite, 1);
      }
    }

    // ---- ROW layout, straight from registers
    if constexpr (ROW) {
      // 1x128: the 16 lanes of a group hold the same 8 row maxima; lane li
      // derives the scale of row li % 8 (one correctly rounded divide pair
      // per lane instead of eight) and the group reads them back by shuffle
      float s_rows[8];
      bool bad_rows[8];
      if constexpr (MODE == MODE_B1x128) {
        uint32_t kk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float v[8];
          cur.row(i, v);
          kk[i] = group_max_u32<16>(cur.key(i, v));
          bad_rows[i] = !is_finite(key_to_float(kk[i]));
        }
        uint32_t kj = kk[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) kj = ((li & 7) == j) ? kk[j] : kj;
        const float amj = key_to_float(kj);
        const float sj = scale_from_amax<FMT>(amj, a.margin);
        const int64_t rj = row0 + g + 16 * (li & 7);
        if (li < 8 && rj < a.rows) {
          reinterpret_cast<float*>(a.s_row)[rj * tiles_x + bx] = recip_rn(sj);
          if (!is_finite(amj) && a.nonfinite) atomicAdd(a.nonfinite, 1);
        }
        const int gbase = (tid & 63) & ~15;
#pragma unroll
        for (int i = 0; i < 8; ++i) s_rows[i] = __shfl(sj, gbase + i, 64);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t r = row0 + g + 16 * i;
        float v[8];
        cur.row(i, v);
        float s = s_t;
        bool safe = safe_t;
        if constexpr (MODE == MODE_B1x128) {
          s = s_rows[i];
          safe = bad_rows[i];
        } else if constexpr (MODE == MODE_MX32 || MODE == MODE_MX32F) {
          const uint32_t k = group_max_u32<4>(cur.key(i, v));
          const int byte = mx_byte<MODE, FMT>(key_to_float(k));
          // the floor rule lets elements exceed max: saturating encoder
          safe = byte == 0xFF || MODE == MODE_MX32F;
          s = byte == 0xFF ? 1.0f : mx_inv_scale(byte);
          if ((li & 3) == 0 && r < a.rows && nval > 0) {
            const int64_t gc = (a.cols + 31) / 32;
            reinterpret_cast<uint8_t*>(a.s_row)[r * gc + (ccol >> 5)] = (uint8_t)byte;
            if (byte == 0xFF && a.nonfinite) atomicAdd(a.nonfinite, 1);
          }
        } else if constexpr (MODE == MODE_TENSOR && !CURRENT) {
          const uint32_t k = cur.key(i, v);
          amax_acc = amax_acc > k ? amax_acc : k;
          safe = !fits<FMT>(k, s);
        } else if constexpr (MODE == MODE_CHANNEL) {
          const float sr = r < a.rows ? reinterpret_cast<const float*>(a.s_row)[r] : 1.0f;
          s = chan_s(sr);
          safe = chan_bad(sr);
        }
        if (r < a.rows && nval > 0) {
          uint2 c = safe ? encode8<FMT, true>(v, s) : encode8<FMT, false>(v, s);
          store8(a.q_row + r * a.ld_q_row + ccol, nval, c);
        }
      }
    }

    // ---- COL layout: transpose through LDS.  The raw rows go to LDS as they
    // were loaded; thread (cp, rq) then walks rows [32 rq, 32 rq + 32) of the
    // column pair (2 cp, 2 cp + 1) with one 4-byte (BF16) or 8-byte (FP32)
    // read per row and encodes 32 codes of each column.
    if constexpr (COL) {
      __syncthreads();  // the previous tile's column pass is done with `tile`
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rl = g + 16 * i;
        if constexpr (sizeof(InT) == 2) {
          reinterpret_cast<uint4*>(tile)[(rl * kTile + 8 * li) / 8] = cur.w[i];
        } else {
          reinterpret_cast<float4*>(tile)[(rl * kTile + 8 * li) / 4] = cur.w[2 * i];
          reinterpret_cast<float4*>(tile)[(rl * kTile + 8 * li) / 4 + 1] = cur.w[2 * i + 1];
        }
      }
      __syncthreads();

      const int cp = tid & 63;  // column pair: tile columns 2cp, 2cp+1
      const int rq = tid >> 6;  // rows 32rq .. 32rq+31 (one wave per quarter)
      const int64_t colA = col0 + 2 * cp;
      const int64_t rbase = row0 + 32 * rq;
      float w0[32], w1[32];
      uint32_t k0 = 0, k1 = 0;  // max |x| keys of the two column segments
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int rl = 32 * rq + j;
        if constexpr (sizeof(InT) == 2) {
          const uint32_t pr = reinterpret_cast<const uint32_t*>(tile)[rl * (kTile / 2) + cp];
          w0[j] = __builtin_bit_cast(float, pr << 16);
          w1[j] = __builtin_bit_cast(float, pr & 0xFFFF0000u);
        } else {
          const float2 pr = reinterpret_cast<const float2*>(tile)[rl * (kTile / 2) + cp];
          w0[j] = pr.x;
          w1[j] = pr.y;
        }
        const uint32_t a0 = abs_key(w0[j]), a1 = abs_key(w1[j]);
        k0 = k0 > a0 ? k0 : a0;
        k1 = k1 > a1 ? k1 : a1;
      }

      float s0 = s_t, s1 = s_t;  // scales of the two columns
      bool safe0 = safe_t, safe1 = safe_t;
      if constexpr (MODE == MODE_TENSOR && !CURRENT) {
        if constexpr (!ROW) {
          const uint32_t m = k0 > k1 ? k0 : k1;
          amax_acc = amax_acc > m ? amax_acc : m;
        }
        safe0 = !fits<FMT>(k0, s_t);
        safe1 = !fits<FMT>(k1, s_t);
      } else if constexpr (MODE == MODE_B1x128) {
        colred[rq][2 * cp] = k0;
        colred[rq][2 * cp + 1] = k1;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          k0 = k0 > colred[q][2 * cp] ? k0 : colred[q][2 * cp];
          k1 = k1 > colred[q][2 * cp + 1] ? k1 : colred[q][2 * cp + 1];
        }
        const float am0 = key_to_float(k0), am1 = key_to_float(k1);
        s0 = scale_from_amax<FMT>(am0, a.margin);
        s1 = scale_from_amax<FMT>(am1, a.margin);
        safe0 = !is_finite(am0);
        safe1 = !is_finite(am1);
        if (rq == 0) {
          const int64_t gr = (a.rows + kTile - 1) / kTile;
          if (colA < a.cols) {
            reinterpret_cast<float*>(a.s_col)[colA * gr + by] = recip_rn(s0);
            if (safe0 && a.nonfinite) atomicAdd(a.nonfinite, 1);
          }
          if (colA + 1 < a.cols) {
            reinterpret_cast<float*>(a.s_col)[(colA + 1) * gr + by] = recip_rn(s1);
            if (safe1 && a.nonfinite) atomicAdd(a.nonfinite, 1);
          }
        }
      } else if constexpr (MODE == MODE_CHANNEL) {
        const float* sc = reinterpret_cast<const float*>(a.s_col);
        const float v0 = colA < a.cols ? sc[colA] : 1.0f, v1 = colA + 1 < a.cols ? sc[colA + 1] : 1.0f;
        s0 = chan_s(v0);
        s1 = chan_s(v1);
        safe0 = chan_bad(v0);
        safe1 = chan_bad(v1);
      } else if constexpr (MODE == MODE_MX32 || MODE == MODE_MX32F) {
        const int b0 = mx_byte<MODE, FMT>(key_to_float(k0));
        const int b1 = mx_byte<MODE, FMT>(key_to_float(k1));
        safe0 = b0 == 0xFF || MODE == MODE_MX32F;
        safe1 = b1 == 0xFF || MODE == MODE_MX32F;
        s0 = b0 == 0xFF ? 1.0f : mx_inv_scale(b0);
        s1 = b1 == 0xFF ? 1.0f : mx_inv_scale(b1);
        if (rbase < a.rows) {
          const int64_t gr = (a.rows + 31) / 32;
          uint8_t* sc = reinterpret_cast<uint8_t*>(a.s_col);
          if (colA < a.cols) {
            sc[colA * gr + (rbase >> 5)] = (uint8_t)b0;
            if (b0 == 0xFF && a.nonfinite) atomicAdd(a.nonfinite, 1);
          }
          if (colA + 1 < a.cols) {
            sc[(colA + 1) * gr + (rbase >> 5)] = (uint8_t)b1;
            if (b1 == 0xFF && a.nonfinite) atomicAdd(a.nonfinite, 1);
          }
        }
      }

      // codes of the two columns, 32 rows each
      uint32_t pk[2][8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float* w = half ? w1 : w0;
        const float s = half ? s1 : s0;
        const bool safe = half ? safe1 : safe0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          pk[half][q] = safe ? encode4<FMT, true>(w[4 * q] * s, w[4 * q + 1] * s, w[4 * q + 2] * s, w[4 * q + 3] * s)
                             : encode4<FMT, false>(w[4 * q] * s, w[4 * q + 1] * s, w[4 * q + 2] * s, w[4 * q + 3] * s);
      }
      // The codes go out through LDS: each thread's 2 x 32 bytes land in a
      // [128 columns x kCodeStride] byte tile that reuses `tile` (every
      // thread is past its reads of it), and are read back so that 8
      // consecutive lanes store one output row's 128 bytes: whole cache
      // lines instead of 16-byte pieces of 64 different rows.
      __syncthreads();
      uint8_t* ct = reinterpret_cast<uint8_t*>(tile);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint4* d = reinterpret_cast<uint4*>(ct + (2 * cp + half) * kCodeStride + 32 * rq);
        d[0] = make_uint4(pk[half][0], pk[half][1], pk[half][2], pk[half][3]);
        d[1] = make_uint4(pk[half][4], pk[half][5], pk[half][6], pk[half][7]);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kTile * kTile / 16 / kThreads; ++k) {
        const int idx = tid + kThreads * k;
        const int c = idx >> 3, m = idx & 7;  // tile column (output row), 16-row chunk
        const int64_t col = col0 + c, r0 = row0 + 16 * m;
        if (col < a.cols && r0 < a.rows) {
          const uint4 v = *reinterpret_cast<const uint4*>(ct + c * kCodeStride + 16 * m);
          uint8_t* dst = a.q_col + col * a.ld_q_col + r0;
          if (r0 + 16 <= a.rows) {
            *reinterpret_cast<uint4*>(dst) = v;
          } else {
            const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
            for (int j = 0; j < a.rows - r0; ++j) dst[j] = (uint8_t)((vw[j >> 2] >> (8 * (j & 3))) & 0xFF);
          }
        }
      }
    }
    cur = nxt;
  }

  if constexpr (MODE == MODE_TENSOR && !CURRENT) {
    const uint32_t k = wg_max_u32(amax_acc, red4);
    if (tid == 0) reinterpret_cast<uint32_t*>(a.amax)[blockIdx.x] = k;
  }
}

// ---------------------------------------------------------------------------
// Per-tensor amax for current scaling: max |x| over the tensor, NaN-dominant.
// Each workgroup of the reduction pass stores its partial maximum (a |x| bit
// pattern) in slot 1 + w of the caller's amax array; every workgroup of the
// cast pass folds the slots itself and workgroup 0 writes amax[0].
// ---------------------------------------------------------------------------
__device__ __forceinline__ void put_partial(uint32_t k, uint32_t* slots) {
  slots[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = k;
}

// max |x| key of 8 consecutive elements (fewer at a ragged row end)
__device__ __forceinline__ uint32_t chunk_key(const uint16_t* p, int64_t n) {
  if (n >= 8) return bf16x8_key(*reinterpret_cast<const uint4*>(p));
  float v[8];
  load8(p, n, v);
  return max8_key(v);
}
__device__ __forceinline__ uint32_t chunk_key(const float* p, int64_t n) {
  float v[8];
  load8(p, n, v);
  return max8_key(v);
}

// Rows stride over blockIdx.y, 8-element chunks of a row over
// blockIdx.x * 256 + tid; four rows per trip keep four loads in flight.
template <typename InT>
__global__ __launch_bounds__(kThreads) void amax_kernel(const InT* x, int64_t rows, int64_t cols,
                                                        int64_t ld, uint32_t* slots) {
  __shared__ uint32_t red4[4];
  const int64_t cpr = (cols + 7) / 8;
  uint32_t k = 0;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cpr; c += (int64_t)gridDim.x * kThreads) {
    const int64_t cc = 8 * c;
    int64_t r = blockIdx.y;
    for (; r + 3 * (int64_t)gridDim.y < rows; r += 4 * (int64_t)gridDim.y) {
      const uint32_t k0 = chunk_key(x + r * ld + cc, cols - cc);
      const uint32_t k1 = chunk_key(x + (r + gridDim.y) * ld + cc, cols - cc);
      const uint32_t k2 = chunk_key(x + (r + 2 * (int64_t)gridDim.y) * ld + cc, cols - cc);
      const uint32_t k3 = chunk_key(x + (r + 3 * (int64_t)gridDim.y) * ld + cc, cols - cc);
      const uint32_t a = k0 > k1 ? k0 : k1, b = k2 > k3 ? k2 : k3;
      const uint32_t m = a > b ? a : b;
      k = k > m ? k : m;
    }
    for (; r < rows; r += gridDim.y) {
      const uint32_t m = chunk_key(x + r * ld + cc, cols - cc);
      k = k > m ? k : m;
    }
  }
  k = wg_max_u32(k, red4);
  if (threadIdx.x == 0) put_partial(k, slots);
}

// Contiguous tensors (ld == cols): one flat stream of 8-element chunks,
// grid-strided with four independent 16-byte loads per trip.
template <typename InT>
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(const InT* x, int64_t n, uint32_t* slots) {
  __shared__ uint32_t red4[4];
  const int64_t nch = n / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t k = 0;
  for (; i + 3 * stride < nch; i += 4 * stride) {
    const uint32_t k0 = chunk_key(x + 8 * i, 8);
    const uint32_t k1 = chunk_key(x + 8 * (i + stride), 8);
    const uint32_t k2 = chunk_key(x + 8 * (i + 2 * stride), 8);
    const uint32_t k3 = chunk_key(x + 8 * (i + 3 * stride), 8);
    const uint32_t a = k0 > k1 ? k0 : k1, b = k2 > k3 ? k2 : k3;
    const uint32_t m = a > b ? a : b;
    k = k > m ? k : m;
  }
  for (; i < nch; i += stride) {
    const uint32_t m = chunk_key(x + 8 * i, 8);
    k = k > m ? k : m;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && n > 8 * nch) {
    const uint32_t m = chunk_key(x + 8 * nch, n - 8 * nch);
    k = k > m ? k : m;
  }
  k = wg_max_u32(k, red4);
  if (threadIdx.x == 0) put_partial(k, slots);
}

// ---------------------------------------------------------------------------
// Channel-wise scaling ("Mastering FP8 LLM training", Fig. 1 discussion: one
// scale per channel, a row or a column): four passes.
//   1. chan_amax_kernel: one workgroup per 128 x 128 tile stores the tile's
//      per-row (ROW) and per-column (COL) max |x| keys as partials laid over
//      the code outputs: row r, tile column bx at q_row[r][4 bx]; column c,
//      tile row by at q_col[c][4 by].  When one tile spans the whole row
//      (column) the scale is final and goes straight to s_row (s_col).
//   2. chan_reduce_kernel: 16 lanes per row (column) fold its partials into
//      the scale s, stored in s_row (s_col), sign bit set for a non-finite
//      amax.
//   3. the tile kernel casts with those scales (MODE_CHANNEL), overwriting
//      the partials with codes.
//   4. chan_finalize_kernel: s -> s_inv in place, counting non-finite rows.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ float chan_encode_scale(uint32_t key, int margin) {
  const float am = key_to_float(key);
  return is_finite(am) ? scale_from_amax<FMT>(am, margin) : -1.0f;
}

template <typename InT, int FMT, bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void chan_amax_kernel(TileArgs a) {
  __shared__ uint32_t colk[16][kTile];
  const int tid = threadIdx.x;
  const int g = tid >> 4, li = tid & 15;
  const int64_t tiles_x = (a.cols + kTile - 1) / kTile, tiles_y = (a.rows + kTile - 1) / kTile;
  const int64_t t = blockIdx.x;
  const int64_t by = t / tiles_x, bx = t - by * tiles_x;
  const int64_t row0 = by * kTile, ccol = bx * kTile + 8 * li;
  Raw<InT> cur;
  cur.load(reinterpret_cast<const InT*>(a.x), a.ld_x, a.rows, row0 + g, ccol, a.cols - ccol);
  uint32_t ck[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // COL: this thread's 8 columns over its 8 rows
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v[8];
    cur.row(i, v);
    if constexpr (ROW) {
      const uint32_t k = group_max_u32<16>(cur.key(i, v));
      const int64_t r = row0 + g + 16 * i;
      if (li == 0 && r < a.rows) {
        if (tiles_x == 1)
          reinterpret_cast<float*>(a.s_row)[r] = chan_encode_scale<FMT>(k, a.margin);
        else
          *reinterpret_cast<uint32_t*>(a.q_row + r * a.ld_q_row + 4 * bx) = k;
      }
    }
    if constexpr (COL) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t k = abs_key(v[e]);  // rows past the edge loaded as 0
        ck[e] = ck[e] > k ? ck[e] : k;
      }
    }
  }
  if constexpr (COL) {
#pragma unroll
    for (int e = 0; e < 8; ++e) colk[g][8 * li + e] = ck[e];
    __syncthreads();
    if (tid < kTile) {
      uint32_t k = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) k = k > colk[q][tid] ? k : colk[q][tid];
      const int64_t c = bx * kTile + tid;
      if (c < a.cols) {
        if (tiles_y == 1)
          reinterpret_cast<float*>(a.s_col)[c] = chan_encode_scale<FMT>(k, a.margin);
        else
          *reinterpret_cast<uint32_t*>(a.q_col + c * a.ld_q_col + 4 * by) = k;
      }
    }
  }
}

// 16 lanes per line (a row of q_row or of q_col): fold n partial keys.
template <int FMT>
__global__ __launch_bounds__(kThreads) void chan_reduce_kernel(const uint8_t* part, int64_t ld, int64_t lines,
                                                               int64_t n, float* s_out, int margin) {
  const int64_t line = (int64_t)blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4);
  const int li = threadIdx.x & 15;
  uint32_t k = 0;
  if (line < lines) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(part + line * ld);
    for (int64_t j = li; j < n; j += 16) k = k > p[j] ? k : p[j];
  }
  k = group_max_u32<16>(k);
  if (li == 0 && line < lines) s_out[line] = chan_encode_scale<FMT>(k, margin);
}

// s -> s_inv over the row scales then the column scales
__global__ __launch_bounds__(kThreads) void chan_finalize_kernel(float* s_row, int64_t n_row, float* s_col,
                                                                 int64_t n_col, int32_t* nonfinite) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float* p = i < n_row ? s_row + i : (i < n_row + n_col ? s_col + (i - n_row) : nullptr);
  if (!p) return;
  const float v = *p;
  *p = recip_rn(chan_s(v));
  if (chan_bad(v) && nonfinite) atomicAdd(nonfinite, 1);
}

// Persistent grid: as many workgroups as stay resident on the stream's device
// (per the kernel's register / LDS occupancy, which depends only on the
// kernel and the architecture), rounded so every workgroup walks the same
// number of tiles.
template <typename Kernel>
unsigned persistent_grid(Kernel k, int64_t tiles, std::atomic<int>& per_cu_cache, hipStream_t st) {
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, 0) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  const int64_t resident = (int64_t)cu_count(stream_device(st)) * per_cu;
  const int64_t rounds = (tiles + resident - 1) / resident;
  return (unsigned)((tiles + rounds - 1) / rounds);
}

template <typename InT, int FMT, int MODE, bool ROW, bool COL, bool CURRENT>
hipError_t launch_tile_k(const TileArgs& a, int64_t tiles, hipStream_t st) {
  static std::atomic<int> occupancy{0};  // workgroups per CU
  auto k = quant_tile_kernel<InT, FMT, MODE, ROW, COL, CURRENT>;
  unsigned grid = persistent_grid(k, tiles, occupancy, st);
  // delayed scaling: one accumulator slot per workgroup
  if (MODE == MODE_TENSOR && !CURRENT && grid > (unsigned)kAmaxSlots) grid = kAmaxSlots;
  k<<<grid, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <typename InT, int FMT, int MODE, bool CURRENT>
hipError_t launch_tile(const QuantParams& p, hipStream_t st, int nparts = 0, const uint32_t* parts = nullptr) {
  TileArgs a{p.x, p.rows, p.cols, p.ld_x, p.q_row, p.ld_q_row, p.s_row, p.q_col, p.ld_q_col,
             p.s_col, p.scale, p.scale_inv, p.amax, p.nonfinite, p.margin, nparts, parts};
  const int64_t tiles = ((p.cols + kTile - 1) / kTile) * ((p.rows + kTile - 1) / kTile);
  const bool row = p.orient & 1, col = p.orient & 2;
  if (row && col) return launch_tile_k<InT, FMT, MODE, true, true, CURRENT>(a, tiles, st);
  if (row) return launch_tile_k<InT, FMT, MODE, true, false, CURRENT>(a, tiles, st);
  return launch_tile_k<InT, FMT, MODE, false, true, CURRENT>(a, tiles, st);
}

template <typename InT, int FMT>
hipError_t launch_fmt(const QuantParams& p, hipStream_t st) {
  switch (p.recipe) {
    case kRecipeTensorCurrent: {
      if (p.rows > 0 && p.cols > 0) {
        const InT* x = reinterpret_cast<const InT*>(p.x);
        // partial maxima: amax[1 .. kAmaxSlots - 1], or the static scratch
        uint32_t* slots = p.partials ? p.partials : reinterpret_cast<uint32_t*>(p.amax) + 1;
        int64_t cap = (int64_t)cu_count(stream_device(st)) * 8;
        cap = cap < kMaxPartials ? cap : kMaxPartials;
        int64_t parts;
        if (p.ld_x == p.cols || p.rows == 1) {
          const int64_t n = p.rows * p.cols;
          int64_t blocks = (n / 8 + kThreads - 1) / kThreads;
          blocks = blocks < cap ? blocks : cap;
          parts = blocks > 0 ? blocks : 1;
          amax_flat_kernel<InT><<<(unsigned)parts, kThreads, 0, st>>>(x, n, slots);
        } else {
          const int64_t cpr = (p.cols + 7) / 8;
          int64_t gx = (cpr + kThreads - 1) / kThreads;
          gx = gx < 64 ? gx : 64;
          gx = gx < cap ? gx : cap;
          int64_t gy = cap / gx;
          gy = gy < p.rows ? gy : p.rows;
          gy = gy < 65535 ? gy : 65535;
          gy = gy > 0 ? gy : 1;
          parts = gx * gy;
          amax_kernel<InT><<<dim3((unsigned)gx, (unsigned)gy), kThreads, 0, st>>>(x, p.rows, p.cols, p.ld_x,
                                                                                  slots);
        }
        return launch_tile<InT, FMT, MODE_TENSOR, true>(p, st, (int)parts, slots);
      }
      // empty tensor: amax = 0 -> scale = scale_inv = 1
      return launch_empty_scale(p.amax, p.scale, p.scale_inv, st);
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
    case kRecipeMx1x32Ocp:
      return launch_tile<InT, FMT, MODE_MX32F, false>(p, st);
    case kRecipeChannel: {
      TileArgs a{p.x, p.rows, p.cols, p.ld_x, p.q_row, p.ld_q_row, p.s_row, p.q_col, p.ld_q_col,
                 p.s_col, p.scale, p.scale_inv, p.amax, p.nonfinite, p.margin, 0, nullptr};
      const bool row = p.orient & 1, col = p.orient & 2;
      const int64_t tx = (p.cols + kTile - 1) / kTile, ty = (p.rows + kTile - 1) / kTile;
      const unsigned tiles = (unsigned)(tx * ty);
      if (row && col)
        chan_amax_kernel<InT, FMT, true, true><<<tiles, kThreads, 0, st>>>(a);
      else if (row)
        chan_amax_kernel<InT, FMT, true, false><<<tiles, kThreads, 0, st>>>(a);
      else
        chan_amax_kernel<InT, FMT, false, true><<<tiles, kThreads, 0, st>>>(a);
      constexpr int kLines = kThreads / 16;
      if (row && tx > 1)
        chan_reduce_kernel<FMT><<<(unsigned)((p.rows + kLines - 1) / kLines), kThreads, 0, st>>>(
            p.q_row, p.ld_q_row, p.rows, tx, reinterpret_cast<float*>(p.s_row), p.margin);
      if (col && ty > 1)
        chan_reduce_kernel<FMT><<<(unsigned)((p.cols + kLines - 1) / kLines), kThreads, 0, st>>>(
            p.q_col, p.ld_q_col, p.cols, ty, reinterpret_cast<float*>(p.s_col), p.margin);
      const hipError_t e = launch_tile<InT, FMT, MODE_CHANNEL, false>(p, st);
      if (e != hipSuccess) return e;
      const int64_t n_row = row ? p.rows : 0, n_col = col ? p.cols : 0;
      chan_finalize_kernel<<<(unsigned)((n_row + n_col + kThreads - 1) / kThreads), kThreads, 0, st>>>(
          reinterpret_cast<float*>(p.s_row), n_row, reinterpret_cast<float*>(p.s_col), n_col, p.nonfinite);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

__global__ void empty_scale_kernel(float* amax, float* scale, float* scale_inv) {
  *amax = 0.0f;
  *scale = 1.0f;
  *scale_inv = 1.0f;
}

}  // namespace

hipError_t launch_empty_scale(float* amax, float* scale, float* scale_inv, hipStream_t st) {
  empty_scale_kernel<<<1, 1, 0, st>>>(amax, scale, scale_inv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (fp8_quantize_static_scratch):
// current scaling's partial maxima live in this file-scope device array, one
// copy per GPU, instead of the caller's amax[1 ..].  Host code never passes
// the array's name to a kernel: it looks up the array's device address once
// per device (with that device current) and passes that.  Every slot the
// cast pass reads is written by the amax pass of the same call first, so the
// array needs no clearing; calls that overlap on one GPU share it and race.
// ---------------------------------------------------------------------------
constexpr int kScratchWords = 1024;
static_assert(kMaxPartials <= kScratchWords, "the amax pass's partial maxima fit the scratch");
static __device__ __align__(256) uint32_t scratch[kScratchWords];

// device address of `scratch` on device dev (nullptr if the lookup failed)
static uint32_t* scratch_address(int dev) {
  static std::atomic<uint32_t*> addr[kMaxDevices];
  static std::mutex lock;
  uint32_t* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> g(lock);
  p = addr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* found = nullptr;
  const hipError_t e = hipGetSymbolAddress(&found, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !found) return nullptr;
  p = static_cast<uint32_t*>(found);
  addr[dev].store(p, std::memory_order_release);
  return p;
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t st) {
  if (p.recipe != kRecipeTensorCurrent && (p.rows == 0 || p.cols == 0)) return hipSuccess;
  if (p.x_dtype == kInBf16) {
    return p.fmt == kE4M3 ? launch_fmt<uint16_t, kE4M3>(p, st) : launch_fmt<uint16_t, kE5M2>(p, st);
  }
  return p.fmt == kE4M3 ? launch_fmt<float, kE4M3>(p, st) : launch_fmt<float, kE5M2>(p, st);
}

hipError_t launch_quantize_static_scratch(const QuantParams& p, hipStream_t st) {
  QuantParams q = p;
  if (p.recipe == kRecipeTensorCurrent && p.rows > 0 && p.cols > 0) {
    q.partials = scratch_address(stream_device(st));
    if (!q.partials) return hipErrorInvalidSymbol;
  }
  return launch_quantize(q, st);
}

}  // namespace fp8mi
