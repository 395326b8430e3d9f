// history.hip -- delayed-scaling amax history update.
//
// "2025 technical guide: FP8 quantized training", sec. 2.1: delayed scaling
// keeps the amax of the past steps (usually 200) in a buffer and derives the
// scale from the buffer's maximum.  "From FP16 to FP8", sec. 3.3: the recipe
// updates every step (interval 1) with a margin (0 there).
//
// One workgroup: fold the accumulator's slots (the per-workgroup maxima the
// delayed-scaling casts left since the last update) into the step's amax,
// push it at `head` if finite, advance the ring, reduce the ring maximum,
// write the next scale and its reciprocal, and re-arm every slot with 0.
// All state is device-resident; there is no host round trip.
#include "device.hpp"
#include "launch.hpp"

namespace fp8mi {

namespace {

constexpr int kHistThreads = 1024;

// One round of loads (a slot and a ring entry per thread), one reduction.
// The ring maximum leaves out entry h, which the step's amax replaces when
// it is pushed and which is folded back in when it is not.
template <int FMT>
__global__ __launch_bounds__(kHistThreads) void history_kernel(float* ring, int32_t* head, int len, float* amax,
                                                               int margin, float* scale, float* scale_inv,
                                                               int32_t* nonfinite) {
  __shared__ uint32_t redk[kHistThreads / 64];
  __shared__ float redr[kHistThreads / 64];
  __shared__ float ring_h;
  uint32_t* slots = reinterpret_cast<uint32_t*>(amax);
  const int t = threadIdx.x;
  // head, slots and ring are all loaded in one round (no load waits on
  // another); the entry at head is picked out afterwards.  A head outside
  // [0, len) (state saved with another length, or corrupted) is taken
  // modulo len, so every ring access stays inside the ring.
  const int h0 = *head % len;
  const int h = h0 < 0 ? h0 + len : h0;
  // the step's amax: NaN-dominant max over the slots (|x| bit patterns)
  uint32_t k = 0;
  for (int i = t; i < kAmaxSlots; i += kHistThreads) {
    const uint32_t v = slots[i];
    k = k > v ? k : v;
  }
  float m = 0.0f;  // ring entries are finite and non-negative
  for (int i = t; i < len; i += kHistThreads) {
    const float r = ring[i];
    if (i != h) m = fmaxf(m, r);
    else ring_h = r;
  }
  k = group_max_u32<64>(k);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((t & 63) == 0) {
    redk[t >> 6] = k;
    redr[t >> 6] = m;
  }
  __syncthreads();  // every slot and ring entry has been read before they are rewritten
  for (int i = t; i < kAmaxSlots; i += kHistThreads) slots[i] = 0u;
  if (t == 0) {
    k = 0;
    m = 0.0f;
#pragma unroll
    for (int w = 0; w < kHistThreads / 64; ++w) {
      k = k > redk[w] ? k : redk[w];
      m = fmaxf(m, redr[w]);
    }
    const float a = key_to_float(k);
    const bool push = is_finite(a);
    m = fmaxf(m, push ? a : ring_h);
    if (push) {
      ring[h] = a;
      *head = (h + 1) % len;
    } else if (nonfinite) {
      *nonfinite += 1;
    }
    const float s = scale_from_amax<FMT>(m, margin);
    *scale = s;
    *scale_inv = recip_rn(s);
  }
}

}  // namespace

hipError_t launch_history(float* history, int32_t* head, int len, float* amax, int fmt, int margin,
                          float* scale, float* scale_inv, int32_t* nonfinite, hipStream_t st) {
  if (fmt == kE4M3)
    history_kernel<kE4M3><<<1, kHistThreads, 0, st>>>(history, head, len, amax, margin, scale, scale_inv, nonfinite);
  else
    history_kernel<kE5M2><<<1, kHistThreads, 0, st>>>(history, head, len, amax, margin, scale, scale_inv, nonfinite);
  return hipGetLastError();
}

}  // namespace fp8mi
