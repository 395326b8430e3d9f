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

template <int FMT>
__global__ __launch_bounds__(256) void history_kernel(float* ring, int32_t* head, int len, float* amax,
                                                      int margin, float* scale, float* scale_inv,
                                                      int32_t* nonfinite) {
  __shared__ uint32_t redk[4];
  __shared__ float red[4];
  // the step's amax: NaN-dominant max over the slots (|x| bit patterns)
  uint32_t* slots = reinterpret_cast<uint32_t*>(amax);
  uint32_t k = 0;
  for (int i = threadIdx.x; i < kAmaxSlots; i += blockDim.x) {
    const uint32_t v = slots[i];
    k = k > v ? k : v;
  }
  k = group_max_u32<64>(k);
  if ((threadIdx.x & 63) == 0) redk[threadIdx.x >> 6] = k;
  const int h = *head;
  __syncthreads();  // every slot and *head have been read before they are rewritten
  const uint32_t k01 = redk[0] > redk[1] ? redk[0] : redk[1];
  const uint32_t k23 = redk[2] > redk[3] ? redk[2] : redk[3];
  const float a = key_to_float(k01 > k23 ? k01 : k23);
  const bool push = is_finite(a);
  float m = push ? a : 0.0f;  // the pushed value replaces ring[h]
  for (int i = threadIdx.x; i < len; i += blockDim.x)
    if (!(push && i == h)) m = fmaxf(m, ring[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  for (int i = threadIdx.x; i < kAmaxSlots; i += blockDim.x) slots[i] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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
    history_kernel<kE4M3><<<1, 256, 0, st>>>(history, head, len, amax, margin, scale, scale_inv, nonfinite);
  else
    history_kernel<kE5M2><<<1, 256, 0, st>>>(history, head, len, amax, margin, scale, scale_inv, nonfinite);
  return hipGetLastError();
}

}  // namespace fp8mi
