// device.hpp -- gfx950 device helpers shared by the quantize, history and
// GEMM kernels: FP8 formats, the saturating nearest-even cast, scale from
// amax, BF16 unpacking and wave reductions.
//
// Formats and scale rule: "2025 technical guide: FP8 quantized training"
// sec. 1.1 (E4M3 / E5M2 bit layouts) and sec. 2.1 (scale from amax);
// "From FP16 to FP8" sec. 1-2 (E5M2 max 57344, bias 15) and sec. 3.3
// (margin); "FP8 training support", "Why FP8?" (a scale maps the tensor's
// range onto the FP8 range).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mi {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

template <int FMT>
struct Fmt;
template <>
struct Fmt<kE4M3> {
  static constexpr float kMax = 448.0f;  // S.1111.110
  static constexpr int kEmax = 8;        // 448 = 1.75 * 2^8
};
template <>
struct Fmt<kE5M2> {
  static constexpr float kMax = 57344.0f;  // S.11110.11
  static constexpr int kEmax = 15;         // 57344 = 1.75 * 2^15
};

constexpr float kFltMax = 3.40282346638528859812e+38f;

__device__ __forceinline__ bool is_finite(float v) { return __builtin_fabsf(v) <= kFltMax; }

// s = fl32(max / amax) * 2^-margin; amax == 0 or non-finite -> 1; +Inf -> FLT_MAX.
// The division is the correctly rounded IEEE binary32 divide.
template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax, int margin) {
  if (!is_finite(amax) || amax == 0.0f) return 1.0f;
  float s = __fdiv_rn(Fmt<FMT>::kMax, amax);
  s = __builtin_ldexpf(s, -margin);
  return s > kFltMax ? kFltMax : s;
}

__device__ __forceinline__ float recip_rn(float s) { return __fdiv_rn(1.0f, s); }

// E8M0 byte for an MX block: smallest e with amax * 2^-e <= max, i.e.
// amax = f * 2^E (f in [1,2)) -> e = E - emax + (f > 1.75); clamped to
// [-127, 127]; amax == 0 -> 127; non-finite -> 0xFF.
template <int FMT>
__device__ __forceinline__ int mx_scale_byte(float amax) {
  if (!is_finite(amax)) return 0xFF;
  if (amax == 0.0f) return 127;
  int E = __builtin_amdgcn_frexp_expf(amax) - 1;       // amax = mant * 2^(E+1), mant in [0.5,1)
  float mant = __builtin_amdgcn_frexp_mantf(amax);     // f = 2 * mant
  int e = E - Fmt<FMT>::kEmax + (mant > 0.875f ? 1 : 0);
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return e + 127;
}

// The OCP microscaling specification's exponent rule: floor(log2(amax)) -
// emax, whatever the significand, so a block whose largest element lies
// above max * 2^e saturates it (zero and non-finite amax as above).
template <int FMT>
__device__ __forceinline__ int mx_scale_byte_floor(float amax) {
  if (!is_finite(amax)) return 0xFF;
  if (amax == 0.0f) return 127;
  int e = __builtin_amdgcn_frexp_expf(amax) - 1 - Fmt<FMT>::kEmax;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return e + 127;
}

// 2^-(byte-127) as a binary32 (byte in [0, 254]); 2^127 .. 2^-127 are all
// representable (2^-127 as a subnormal).
__device__ __forceinline__ float mx_inv_scale(int byte) {
  return __builtin_ldexpf(1.0f, 127 - byte);
}

// ---------------------------------------------------------------------------
// FP8 cast on v_cvt_pk_{fp8,bf8}_f32.  The convert rounds to nearest-even in
// the OCP formats, including subnormals, but does not saturate: E4M3 turns
// |v| >= 464 into a NaN code and E5M2 turns |v| >= 61440 into Inf, and every
// NaN input becomes 0xFF (E4M3) / 0xFE (E5M2).  Hence:
//   Safe = false  inputs are finite and at most max * (1 + 2^-22) in
//                 magnitude (scale from a finite amax, or an exact MX power of
//                 two); the convert alone rounds them correctly.
//   Safe = true   any input: v_med3 clamps to [-max, max] (which also maps
//                 +-Inf to +-max) and NaN is routed to the canonical code 0x7F:
//                 E4M3 through a positive overflow sentinel (converts to 0x7F),
//                 E5M2 by rewriting its NaN code 0xFE to 0x7F after packing
//                 (0xFE cannot come from a clamped finite input).
// ---------------------------------------------------------------------------
template <int FMT, bool Safe>
__device__ __forceinline__ float prep(float v) {
  if constexpr (!Safe) {
    return v;
  } else {
    float c = __builtin_amdgcn_fmed3f(v, -Fmt<FMT>::kMax, Fmt<FMT>::kMax);
    if constexpr (FMT == kE4M3)
      return (v != v) ? 1024.0f : c;
    else
      return (v != v) ? v : c;
  }
}

template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old) {
  if constexpr (FMT == kE4M3)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Per byte of w: 0x80 where the byte equals 0xFE, else 0 (carry-free).
__device__ __forceinline__ uint32_t bytes_eq_fe(uint32_t w) {
  uint32_t t = w ^ 0xFEFEFEFEu;
  uint32_t nz = (((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t) & 0x80808080u;
  return ~nz & 0x80808080u;
}

// 4 floats -> 4 codes packed little-endian in one dword.
template <int FMT, bool Safe>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  uint32_t w = cvt2<FMT, false>(prep<FMT, Safe>(a), prep<FMT, Safe>(b), 0u);
  w = cvt2<FMT, true>(prep<FMT, Safe>(c), prep<FMT, Safe>(d), w);
  if constexpr (Safe && FMT == kE5M2) {
    uint32_t m = bytes_eq_fe(w);
    w ^= (m >> 7) * 0x81u;  // 0xFE -> 0x7F
  }
  return w;
}

// ---------------------------------------------------------------------------
// BF16 / FP32 loading: 8 consecutive elements as floats.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack_bf16x8(uint4 w, float v[8]) {
  v[0] = __builtin_bit_cast(float, w.x << 16);
  v[1] = __builtin_bit_cast(float, w.x & 0xFFFF0000u);
  v[2] = __builtin_bit_cast(float, w.y << 16);
  v[3] = __builtin_bit_cast(float, w.y & 0xFFFF0000u);
  v[4] = __builtin_bit_cast(float, w.z << 16);
  v[5] = __builtin_bit_cast(float, w.z & 0xFFFF0000u);
  v[6] = __builtin_bit_cast(float, w.w << 16);
  v[7] = __builtin_bit_cast(float, w.w & 0xFFFF0000u);
}

// |x| as an unsigned key: non-negative floats order like their bit patterns
// and every NaN key exceeds +Inf, so an integer max propagates NaN.
__device__ __forceinline__ uint32_t abs_key(float v) {
  return __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu;
}
__device__ __forceinline__ float key_to_float(uint32_t k) { return __builtin_bit_cast(float, k); }

// ---------------------------------------------------------------------------
// Wave64 reductions (unsigned max) over aligned groups of W lanes.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace fp8mi
