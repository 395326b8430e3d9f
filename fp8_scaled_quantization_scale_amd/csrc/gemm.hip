// gemm.hip -- scaled FP8 GEMMs on gfx950 matrix cores.
//
// "2025 technical guide: FP8 quantized training", sec. 3.1: the three GEMMs of
// a linear layer (fprop, dgrad, wgrad) take quantized inputs and keep
// BF16/FP32 outputs; sec. 2.1-2.3 give the scale granularities; "Mastering
// FP8 LLM training", Fig. 1 discussion: per-block scale factors are applied
// inside the GEMM, which is what makes finer granularity cost throughput.
//
// C[M x N] = dequant(A[M x K]) . dequant(B[N x K])^T, both operands K-contiguous.
//
// Matrix core: v_mfma_f32_16x16x128_f8f6f4 (E4M3 or E5M2 per operand) and its
// block-scaled form v_mfma_scale_f32_16x16x128_f8f6f4 for MX.  Operand layout
// of one 16 x 128 fragment: lane l holds row l % 16; lane group g = l / 16
// holds K bytes [16g, 16g+16) in its first four VGPRs and [64+16g, 64+16g+16)
// in the last four; K block g (bytes [32g, 32g+32)) takes its E8M0 scale from
// lane group g.  Result: lane l, register r holds C[4(l/16) + r][l % 16].
//
// Tiling: 256 threads = 2 x 2 waves, wave tile WM x WN, workgroup tile
// (2 WM) x (2 WN), K step 128 (= one block of the 1x128 / 128x128 recipes,
// = four MX blocks).  A and B tiles are double-buffered in LDS; 16-byte
// chunks are XOR-swizzled by row so the 16 rows read by one lane group hit
// distinct banks.  The next K step's global loads are issued before the
// current step's MFMAs.
//
// Scale application:
//   TENSOR      one alpha = s_a * s_b on the FP32 accumulator at the end;
//   MX          E8M0 scales fed to the scaled MFMA (no VALU work);
//   BLOCK_*     each 128-deep K block is an MFMA into a zeroed FP32 partial,
//               then acc += (s_a[row, kb] * s_b[.., kb]) * partial on the VALU.
#include "device.hpp"
#include "launch.hpp"

namespace fp8mi {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;
constexpr int kThreads = 256;

template <int FA, int FB>
__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz / blgp select the operand formats: 0 = E4M3, 1 = E5M2
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

template <int FA, int FB>
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

struct GArgs {
  const uint8_t* a;
  const uint8_t* b;
  const void* sa;
  const void* sb;
  int64_t lda, ldb, ldc;
  int M, N, K;
  void* c;
  int tiles_m, tiles_n;
};

// LDS byte offset of logical 16-byte chunk `ch` (0..7) of tile row `row`.
__device__ __forceinline__ int swz(int row, int ch) { return row * kBK + ((ch ^ (row & 7)) << 4); }

template <int FA, int FB, int REC, int OUT, int WM, int WN>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GArgs p) {
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int MT = WM / 16, NT = WN / 16;
  constexpr int A_LD = BM * 8 / kThreads;  // 16-byte chunks per thread per K step
  constexpr int B_LD = BN * 8 / kThreads;
  constexpr bool kBlock = REC == kGemmBlock128x128 || REC == kGemmBlock1x128;
  constexpr int SA_N = (REC == kGemmTensor) ? 1 : BM;  // staged A scales per K step
  constexpr int SB_N = (REC == kGemmTensor) ? 1 : (REC == kGemmBlock128x128 ? (BN + 127) / 128 : BN);

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kBK];
  __shared__ __attribute__((aligned(16))) uint32_t lds_sa[2][SA_N];  // float bits or 4 E8M0 bytes
  __shared__ __attribute__((aligned(16))) uint32_t lds_sb[2][SB_N];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15;  // fragment row
  const int lg = lane >> 4;  // lane group

  // ---- tile assignment: XCD-contiguous ranges, then grouped along M
  int pid = blockIdx.x;
  const int total = p.tiles_m * p.tiles_n;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * p.tiles_n;
  const int first_m = (pid / in_group) * GROUP_M;
  const int gsize = min(p.tiles_m - first_m, GROUP_M);
  const int pm = first_m + (pid % in_group) % gsize;
  const int pn = (pid % in_group) / gsize;
  const int m0 = pm * BM, n0 = pn * BN;

  const int KT = (p.K + kBK - 1) / kBK;

  // ---- staging registers for the next K step
  uint4 ra[A_LD], rb[B_LD];
  uint32_t rsa = 0, rsb = 0;

  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + kThreads * i;
      const int row = q >> 3, ch = q & 7;
      const int gm = m0 + row, gk = k0 + 16 * ch;
      ra[i] = (gm < p.M && gk < p.K) ? *reinterpret_cast<const uint4*>(p.a + (int64_t)gm * p.lda + gk)
                                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int q = tid + kThreads * i;
      const int row = q >> 3, ch = q & 7;
      const int gn = n0 + row, gk = k0 + 16 * ch;
      rb[i] = (gn < p.N && gk < p.K) ? *reinterpret_cast<const uint4*>(p.b + (int64_t)gn * p.ldb + gk)
                                     : make_uint4(0, 0, 0, 0);
    }
    if constexpr (kBlock) {
      const int kb = kt;  // one 128-deep K block per step
      const int nkb = KT;
      if (tid < SA_N) {
        const int gm = m0 + tid;
        rsa = gm < p.M ? reinterpret_cast<const uint32_t*>(p.sa)[(int64_t)gm * nkb + kb] : 0u;
      }
      if (tid < SB_N) {
        if constexpr (REC == kGemmBlock128x128) {
          const int gnb = n0 / 128 + tid;
          rsb = gnb * 128 < p.N ? reinterpret_cast<const uint32_t*>(p.sb)[(int64_t)gnb * nkb + kb] : 0u;
        } else {
          const int gn = n0 + tid;
          rsb = gn < p.N ? reinterpret_cast<const uint32_t*>(p.sb)[(int64_t)gn * nkb + kb] : 0u;
        }
      }
    } else if constexpr (REC == kGemmMx) {
      // 4 E8M0 bytes (K blocks 4kt .. 4kt+3) per row, from a [rows x ceil(K/32)] byte grid
      const int nkb = (p.K + 31) / 32;
      const int kb0 = kt * 4;
      if (tid < SA_N) {
        const int gm = m0 + tid;
        uint32_t w = 0x7F7F7F7Fu;
        if (gm < p.M) {
          const uint8_t* s = reinterpret_cast<const uint8_t*>(p.sa) + (int64_t)gm * nkb;
          w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) w |= (uint32_t)(kb0 + j < nkb ? s[kb0 + j] : 127) << (8 * j);
        }
        rsa = w;
      }
      if (tid < SB_N) {
        const int gn = n0 + tid;
        uint32_t w = 0x7F7F7F7Fu;
        if (gn < p.N) {
          const uint8_t* s = reinterpret_cast<const uint8_t*>(p.sb) + (int64_t)gn * nkb;
          w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) w |= (uint32_t)(kb0 + j < nkb ? s[kb0 + j] : 127) << (8 * j);
        }
        rsb = w;
      }
    }
  };

  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&lds_a[st][swz(q >> 3, q & 7)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int q = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&lds_b[st][swz(q >> 3, q & 7)]) = rb[i];
    }
    if constexpr (REC != kGemmTensor) {
      if (tid < SA_N) lds_sa[st][tid] = rsa;
      if (tid < SB_N) lds_sb[st][tid] = rsb;
    }
  };

  // fragment loads: two 16-byte chunks (lane group g: chunks g and 4 + g)
  auto frag = [&](const uint8_t* base, int row) -> v8i {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, lg));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, 4 + lg));
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
  };

  v4f acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (KT > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);

    const uint8_t* la = lds_a[st];
    const uint8_t* lb = lds_b[st];
    v8i fa[MT], fb[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i) fa[i] = frag(la, wm * WM + i * 16 + lr);
#pragma unroll
    for (int j = 0; j < NT; ++j) fb[j] = frag(lb, wn * WN + j * 16 + lr);

    if constexpr (REC == kGemmTensor) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma<FA, FB>(fa[i], fb[j], acc[i][j]);
    } else if constexpr (REC == kGemmMx) {
      int sa[MT], sb[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) sa[i] = (int)((lds_sa[st][wm * WM + i * 16 + lr] >> (8 * lg)) & 0xFFu);
#pragma unroll
      for (int j = 0; j < NT; ++j) sb[j] = (int)((lds_sb[st][wn * WN + j * 16 + lr] >> (8 * lg)) & 0xFFu);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma_mx<FA, FB>(fa[i], fb[j], acc[i][j], sa[i], sb[j]);
    } else {
      // per-row A scales of this lane's four result rows
      float sa[MT][4];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const uint4 w = *reinterpret_cast<const uint4*>(&lds_sa[st][wm * WM + i * 16 + 4 * lg]);
        sa[i][0] = __builtin_bit_cast(float, w.x);
        sa[i][1] = __builtin_bit_cast(float, w.y);
        sa[i][2] = __builtin_bit_cast(float, w.z);
        sa[i][3] = __builtin_bit_cast(float, w.w);
      }
      if constexpr (REC == kGemmBlock128x128) {
        // the wave's WN columns lie inside one 128-wide B tile
        const float sbv = __builtin_bit_cast(float, lds_sb[st][(wn * WN) / 128]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) sa[i][r] *= sbv;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const v4f part = mfma<FA, FB>(fa[i], fb[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[r], sa[i][r], acc[i][j][r]);
          }
      } else {
        float sb[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) sb[j] = __builtin_bit_cast(float, lds_sb[st][wn * WN + j * 16 + lr]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const v4f part = mfma<FA, FB>(fa[i], fb[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(part[r], sa[i][r] * sb[j], acc[i][j][r]);
          }
      }
    }

    if (kt + 1 < KT) sstore(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  float alpha = 1.0f;
  if constexpr (REC == kGemmTensor) {
    if (KT > 0) alpha = *reinterpret_cast<const float*>(p.sa) * *reinterpret_cast<const float*>(p.sb);
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int col = n0 + wn * WN + j * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * WM + i * 16 + 4 * lg + r;
        const float v = (REC == kGemmTensor) ? acc[i][j][r] * alpha : acc[i][j][r];
        if (row < p.M && col < p.N) {
          if constexpr (OUT == kOutBf16)
            reinterpret_cast<__bf16*>(p.c)[(int64_t)row * p.ldc + col] = (__bf16)v;
          else
            reinterpret_cast<float*>(p.c)[(int64_t)row * p.ldc + col] = v;
        }
      }
    }
}

template <int FA, int FB, int REC, int OUT>
hipError_t launch4(const GemmParams& g, hipStream_t st) {
  constexpr bool kBlock = REC == kGemmBlock128x128 || REC == kGemmBlock1x128;
  constexpr int WM = kBlock ? 64 : 128;
  constexpr int WN = 128;
  constexpr int BM = 2 * WM, BN = 2 * WN;
  GArgs a;
  a.a = g.a;
  a.b = g.b;
  a.sa = g.s_a;
  a.sb = g.s_b;
  a.lda = g.lda;
  a.ldb = g.ldb;
  a.ldc = g.ldc;
  a.M = (int)g.M;
  a.N = (int)g.N;
  a.K = (int)g.K;
  a.c = g.c;
  a.tiles_m = (int)((g.M + BM - 1) / BM);
  a.tiles_n = (int)((g.N + BN - 1) / BN);
  const unsigned blocks = (unsigned)a.tiles_m * (unsigned)a.tiles_n;
  gemm_kernel<FA, FB, REC, OUT, WM, WN><<<blocks, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_fmt(const GemmParams& g, hipStream_t st) {
  const bool bf = g.c_dtype == kOutBf16;
  switch (g.recipe) {
    case kGemmTensor:
      return bf ? launch4<FA, FB, kGemmTensor, kOutBf16>(g, st) : launch4<FA, FB, kGemmTensor, kOutFp32>(g, st);
    case kGemmBlock128x128:
      return bf ? launch4<FA, FB, kGemmBlock128x128, kOutBf16>(g, st)
                : launch4<FA, FB, kGemmBlock128x128, kOutFp32>(g, st);
    case kGemmBlock1x128:
      return bf ? launch4<FA, FB, kGemmBlock1x128, kOutBf16>(g, st)
                : launch4<FA, FB, kGemmBlock1x128, kOutFp32>(g, st);
    case kGemmMx:
      return bf ? launch4<FA, FB, kGemmMx, kOutBf16>(g, st) : launch4<FA, FB, kGemmMx, kOutFp32>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const GemmParams& g, hipStream_t st) {
  if (g.fmt_a == kE4M3)
    return g.fmt_b == kE4M3 ? launch_fmt<kE4M3, kE4M3>(g, st) : launch_fmt<kE4M3, kE5M2>(g, st);
  return g.fmt_b == kE4M3 ? launch_fmt<kE5M2, kE4M3>(g, st) : launch_fmt<kE5M2, kE5M2>(g, st);
}

}  // namespace fp8mi
