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
// Data movement: the K loop runs over 128-deep steps (one block of the 1x128 /
// 128x128 recipes, four MX blocks).  Operand tiles stream HBM -> LDS with
// buffer_load_dwordx4 ... lds (no VGPR staging): each wave instruction fills
// 1 KB = 8 tile rows; the lanes fetch permuted 16-byte chunks so that LDS
// holds every row XOR-swizzled (chunk c of row r at slot c ^ swz(r)), which
// keeps the rows one fragment read touches on distinct banks.  Rows past
// the matrix and K past its end come back as zeros from the buffer's range
// check, so the loop has no bounds branches.  A ring of STAGES LDS buffers
// keeps STAGES - 1 steps of loads in flight behind the MFMAs, with one
// workgroup barrier per step.
//
// The same kernel, with BF16 operands and v_mfma_f32_16x16x32_bf16, is the
// BF16 GEMM FP8's speedup is measured against ("Mastering FP8 LLM training",
// Fig. 1): a 128-byte K step is 64 BF16 elements, the two 16-byte halves of a
// fragment feed two 32-deep products, and tiles, data movement and epilogue
// are shared, so the two differ only in the matrix-core instruction.
//
// Scale application:
//   TENSOR      one alpha = s_a * s_b on the FP32 accumulator at the end;
//   CHANNEL     s_a[row] * s_b[col] on the FP32 accumulator at the end;
//   MX          E8M0 scales fed to the scaled MFMA (no VALU work);
//   BLOCK_*     each 128-deep K block is an MFMA into a zeroed FP32 partial,
//               then acc += (s_a[row, kb] * s_b[.., kb]) * partial on the VALU.
#include <utility>

#include "device.hpp"
#include "launch.hpp"

namespace fp8mi {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 128;
constexpr uint32_t kOOB = 0x80000000u;  // voffset past every buffer's range

template <int FA, int FB>
__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz / blgp select the operand formats: 0 = E4M3, 1 = E5M2
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// BF16 operands: the 32-byte fragment holds K elements [8g, 8g+8) and
// [32+8g, 32+8g+8) of lane group g; A and B use the same lane -> K map, so
// two 32-deep products cover the 64-deep step.
__device__ __forceinline__ v4f mfma_bf16(const v8i& a, const v8i& b, v4f c) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i a0 = {a[0], a[1], a[2], a[3]}, a1 = {a[4], a[5], a[6], a[7]};
  const v4i b0 = {b[0], b[1], b[2], b[3]}, b1 = {b[4], b[5], b[6], b[7]};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v8bf, b0), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v8bf, b1), c, 0, 0, 0);
}

// MX tile step: acc[i][j] += B-fragment j x A-fragment i (the C^T form) with
// E8M0 scales.  Lane scale words hold one byte per sub-tile: A sub-tile i in
// byte i % 4 of sa[i / 4], B sub-tile j in byte j % 4 of sb[j / 4]; op_sel
// picks the byte, so the pack is expanded at compile time.
// (one M sub-tile I against all NT B sub-tiles)
template <int FA, int FB, int MT, int NT, int I, int... J>
__device__ __forceinline__ void mx_row(std::integer_sequence<int, J...>, v4f (&acc)[MT][NT], const v8i& fa,
                                       const v8i (&fb)[NT], const uint32_t* sa, const uint32_t* sb) {
  ((acc[I][J] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[J], fa, acc[I][J], FB, FA, J % 4,
                                                                  (int)sb[J / 4], I % 4, (int)sa[I / 4])),
   ...);
}
// All M sub-tiles in order; the A fragment of sub-tile I + 1 is read while
// sub-tile I computes (load_fa), and each sub-tile is its own scheduling
// region, so two A fragments are live at a time.
template <int FA, int FB, int MT, int NT, class LoadFa, int... I>
__device__ __forceinline__ void mx_rows(std::integer_sequence<int, I...>, LoadFa&& load_fa, v4f (&acc)[MT][NT],
                                        const v8i (&fa)[MT], const v8i (&fb)[NT], const uint32_t* sa,
                                        const uint32_t* sb) {
  ((load_fa(I + 1 < MT ? I + 1 : -1),
    mx_row<FA, FB, MT, NT, I>(std::make_integer_sequence<int, NT>{}, acc, fa[I], fb, sa, sb),
    __builtin_amdgcn_sched_barrier(0)),
   ...);
}

// LDS chunk swizzles (16-byte chunk c of tile row r lives at slot c ^ swz(r)).
// A fragments read 16 consecutive rows; B fragments read rows
// 16 g' + 4 j + (0..3) for g' = 0..3 (see brow).  Each 8-lane phase of a
// 16-byte LDS read must see 8 distinct slots: rows r..r+7 for A, bits 0, 1
// and 4 of the row for B.
__device__ __forceinline__ int swz_a(int row) { return row & 7; }
__device__ __forceinline__ int swz_b(int row) { return (row & 3) | ((row >> 2) & 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One wave-wide 16-byte-per-lane LDS DMA: LDS[m0 + 16 * lane] = buffer[voff + soff].
// Issued as inline asm so that the compiler's wait-count pass does not treat
// it as an LDS store aliasing every later LDS read (which would force a full
// vmcnt(0) drain before each K step's fragment reads and serialise the
// prefetch); completion is tracked explicitly with wait_vmcnt below.  The
// s_nop covers the M0-write -> LDS-DMA wait state.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, uint32_t voff,
                                      uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}

// s_waitcnt vmcnt(n) leaving lgkmcnt / expcnt unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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

template <int REC>
struct ScaleTraits {
  // dwords staged per K step for A and for B (float bits or 4 packed E8M0
  // bytes).  2-D A tiles need BM / 128 words, padded to a whole wave so that
  // B's words start on a wave boundary (the padding reads past the grid: zero).
  static constexpr bool kNone = REC == kGemmTensor || REC == kGemmBf16 || REC == kGemmChannel;
  template <int BM>
  static constexpr int a_words() { return kNone ? 0 : (REC == kGemmBlock2d ? 64 : BM); }
  template <int BN>
  static constexpr int b_words() {
    return kNone ? 0 : ((REC == kGemmBlock128x128 || REC == kGemmBlock2d) ? (BN + 127) / 128 : BN);
  }
};

// Tile configuration (measured on MI355X): every recipe runs 256x256
// workgroup tiles with 8 waves of 128x64, two waves per SIMD hiding each
// other's LDS waits.  The block recipes fit it because their A fragments are
// read one M sub-tile ahead inside the promotion pipeline (two live instead
// of eight); MX because a lane's E8M0 scales for a K step fit three
// registers (op_sel picks the byte).  256x128 tiles cost the block recipes
// 11-32% (more LDS and DMA traffic per flop).
template <int REC>
struct TileCfg {
  static constexpr int BM = 256;
  static constexpr int BN = 256;
  static constexpr int WAVES_M = 2;
  static constexpr int WAVES_N = 4;
};

template <int FA, int FB, int REC, int OUT, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_kernel(GArgs p) {
  constexpr int NTHR = 64 * WAVES_M * WAVES_N;
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MT = WM / 16, NT = WN / 16;
  constexpr int SEG_A = BM / 8, SEG_B = BN / 8;  // 1 KB LDS segments per tile
  static_assert((SEG_A + SEG_B) % NWAVES == 0, "segments split evenly over waves");
  constexpr int LOADS = (SEG_A + SEG_B) / NWAVES;  // DMA instructions per wave per K step
  constexpr int TILE_BYTES = (BM + BN) * kBK;
  constexpr int SA_W = ScaleTraits<REC>::template a_words<BM>();
  constexpr int SB_W = ScaleTraits<REC>::template b_words<BN>();
  constexpr int S_W = SA_W + SB_W;
  constexpr bool kBlock = REC == kGemmBlock128x128 || REC == kGemmBlock1x128 || REC == kGemmBlock2d;
  constexpr bool kTileB = REC == kGemmBlock128x128 || REC == kGemmBlock2d;  // B scales per 128x128 tile

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * TILE_BYTES];
  constexpr bool kMx = REC == kGemmMx;
  // block recipes: FP32 scale words of a K step (A rows, then B rows / tiles;
  // every thread stores a word, zeros past S_W)
  constexpr int SLW = S_W > 0 ? (S_W + NTHR - 1) / NTHR : 0;  // scale words per thread
  __shared__ __attribute__((aligned(16))) uint32_t sscale[STAGES][(S_W > 0 && !kMx) ? SLW * NTHR : 1];
  // MX: E8M0 bytes of a K step by K block g: A at [g * BM + pos_a], B at
  // [4 BM + g * BN + pos_b], ordered so that a lane's sub-tile scales are
  // consecutive (see mx_pos_a / mx_pos_b)
  __shared__ __attribute__((aligned(16))) uint8_t sbytes[STAGES][kMx ? 4 * (BM + BN) : 1];

  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lr = lane & 15;  // fragment row
  const int lg = lane >> 4;  // lane group

  // ---- persistent: the workgroup walks tiles blockIdx.x, blockIdx.x +
  // gridDim.x, ... (tiles t and t + gridDim.x stay on one XCD when
  // gridDim.x % 8 == 0); one tile's output stores drain while the next
  // tile's loads and MFMAs run
  const int total = p.tiles_m * p.tiles_n;
#pragma unroll 1
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
  __syncthreads();  // every wave is done with the previous tile's LDS stages
  // ---- tile assignment: XCD-contiguous ranges of the tile index, grouped along M
  int pid = tile;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * p.tiles_n;
  const int first_m = (pid / in_group) * GROUP_M;
  const int gsize = min(p.tiles_m - first_m, GROUP_M);
  const int pm = first_m + (pid % in_group) % gsize;
  const int pn = (pid % in_group) / gsize;
  const int m0 = pm * BM, n0 = pn * BN;
  const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
  const int KT = (p.K + kBK - 1) / kBK;

  // ---- buffer resources over this workgroup's row panels of A and B
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.lda, (uint32_t)(rows_a * p.lda));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (int64_t)n0 * p.ldb, (uint32_t)(rows_b * p.ldb));

  // per-lane source offsets of this wave's DMA segments (K step 0)
  uint32_t voff[LOADS];
  int kchunk[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int seg = wave * LOADS + i;
    const int rsub = lane >> 3;  // row within the 8-row segment
    if (seg < SEG_A) {
      const int row = 8 * seg + rsub;
      const int c = (lane & 7) ^ swz_a(row);  // logical chunk this lane fetches
      kchunk[i] = 16 * c;
      voff[i] = (uint32_t)(row * p.lda + 16 * c);
    } else {
      const int row = 8 * (seg - SEG_A) + rsub;
      const int c = (lane & 7) ^ swz_b(row);
      kchunk[i] = 16 * c;
      voff[i] = (uint32_t)(row * p.ldb + 16 * c);
    }
  }

  // ---- scales: fetched with range-checked buffer loads (zero past the matrix)
  // into VGPRs before a step's tile DMAs, written to LDS at the end of the
  // iteration; every lane issues the same count so vmcnt stays uniform
  // scale words of SB consecutive K steps (see load_scales)
  constexpr int SB = (REC == kGemmBlock1x128) ? 1 : (REC == kGemmMx ? 8 : 4);
  uint32_t rs[SLW > 0 ? SLW : 1][SB];
  __amdgpu_buffer_rsrc_t rsa = make_rsrc(nullptr, 0), rsb = make_rsrc(nullptr, 0);
  int nkb = 0;
  if constexpr (kBlock) {
    nkb = KT;
    if constexpr (REC == kGemmBlock2d)
      rsa = make_rsrc(reinterpret_cast<const uint32_t*>(p.sa) + (int64_t)(m0 / 128) * nkb,
                      (uint32_t)(((rows_a + 127) / 128) * nkb * 4));
    else
      rsa = make_rsrc(reinterpret_cast<const uint32_t*>(p.sa) + (int64_t)m0 * nkb, (uint32_t)(rows_a * nkb * 4));
    if constexpr (kTileB) {
      const int tb = (rows_b + 127) / 128;
      rsb = make_rsrc(reinterpret_cast<const uint32_t*>(p.sb) + (int64_t)(n0 / 128) * nkb, (uint32_t)(tb * nkb * 4));
    } else {
      rsb = make_rsrc(reinterpret_cast<const uint32_t*>(p.sb) + (int64_t)n0 * nkb, (uint32_t)(rows_b * nkb * 4));
    }
  } else if constexpr (REC == kGemmMx) {
    nkb = (p.K + 31) / 32;
    rsa = make_rsrc(reinterpret_cast<const uint8_t*>(p.sa) + (int64_t)m0 * nkb, (uint32_t)(rows_a * nkb));
    rsb = make_rsrc(reinterpret_cast<const uint8_t*>(p.sb) + (int64_t)n0 * nkb, (uint32_t)(rows_b * nkb));
  }

  // A words come first and fill whole waves, so each wave reads one matrix's
  // scales through one (scalar) buffer resource
  static_assert(SA_W % 64 == 0, "A scale words end on a wave boundary");
  // A step's scale word of a row is 4 bytes, and the rows of a panel lie
  // nkb words (bytes for MX) apart, so a per-step fetch is one small request
  // per row.  Where each row's words split evenly into groups of SB steps,
  // 16-byte fetches bring SB steps at once and the words wait in registers,
  // moving down one slot per step (MX GEMMs +5-8%; 1x128 x 1x128 keeps one
  // step per fetch: it has no registers to spare).
  const bool batched = SB > 1 && (kBlock ? (nkb % SB == 0) : (nkb % (4 * SB) == 0));
  auto load_scales = [&](int kt) {
#pragma unroll
    for (int i = 0; i < SLW; ++i) {
      const int t = tid + NTHR * i;
      const bool isa = 64 * wave + NTHR * i < SA_W;  // wave-uniform
      const int r = isa ? t : t - SA_W;  // row (or 128-row tile) within the panel
      const __amdgpu_buffer_rsrc_t rsrc = isa ? rsa : rsb;
      if constexpr (SB > 1) {
        if (batched) {
          if (kt % SB == 0) {  // steps kt .. kt + SB - 1, inside the row
            const uint32_t off = (t < S_W) ? (uint32_t)(kBlock ? (r * nkb + kt) * 4 : r * nkb + 4 * kt) : kOOB;
            typedef int v4i __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int h = 0; h < SB / 4; ++h) {
              const v4i w = __builtin_bit_cast(
                  v4i, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off == kOOB ? kOOB : off + 16 * h, 0, 0));
#pragma unroll
              for (int q = 0; q < 4; ++q) rs[i][4 * h + q] = (uint32_t)w[q];
            }
          }
          continue;
        }
      }
      if constexpr (kBlock) {
        const uint32_t off = (t < S_W) ? (uint32_t)((r * nkb + kt) * 4) : kOOB;
        rs[i][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
      } else if constexpr (REC == kGemmMx) {
        if ((nkb & 3) == 0) {  // the step's 4 bytes are one aligned dword
          const uint32_t off = (t < S_W) ? (uint32_t)(r * nkb + 4 * kt) : kOOB;
          rs[i][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
        } else {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kb = 4 * kt + j;
            const uint32_t off = (t < S_W && kb < nkb) ? (uint32_t)(r * nkb + kb) : kOOB;
            w |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsrc, off, 0, 0) << (8 * j);
          }
          rs[i][0] = w;
        }
      }
    }
  };
  // MX byte positions: A row r = wm WM + 16 i + lr goes to wm WM + lr MT + i;
  // B row r = wn WN + brow(j) (lr = 4 (w / CPL) + w % 4, j = (w % CPL) / 4
  // with w = r % WN) goes to wn WN + lr NT + j
  auto mx_pos_a = [&](int r) {
    const int w = r % WM;
    return (r - w) + (w % 16) * MT + w / 16;
  };
  auto mx_pos_b = [&](int r) {
    constexpr int CPLB = 4 * NT;
    const int w = r % WN;
    return (r - w) + (4 * (w / CPLB) + w % 4) * NT + (w % CPLB) / 4;
  };
  auto store_scales = [&](int kt) {
#pragma unroll
    for (int i = 0; i < SLW; ++i) {
      const int t = tid + NTHR * i;
      if constexpr (kMx) {
        // branch-free (every thread owns a row), so the K step stays one
        // scheduling region
        static_assert(S_W == SLW * NTHR, "one scale row per thread");
        const bool isa = 64 * wave + NTHR * i < SA_W;  // wave-uniform
        const int base = isa ? mx_pos_a(t) : 4 * BM + mx_pos_b(t - SA_W);
        const int gstride = isa ? BM : BN;
        uint8_t* dst = sbytes[kt % STAGES] + base;
        const uint32_t w = rs[i][0];
#pragma unroll
        for (int g = 0; g < 4; ++g) dst[g * gstride] = (uint8_t)(w >> (8 * g));
      } else {
        sscale[kt % STAGES][t] = rs[i][0];  // branch-free: keeps the K step one scheduling region
      }
      // the next step's word moves to slot 0 (a per-step fetch refills it)
#pragma unroll
      for (int q = 0; q + 1 < (int)(sizeof(rs[i]) / sizeof(rs[i][0])); ++q) rs[i][q] = rs[i][q + 1];
    }
  };

  auto issue = [&](int kt) {
    const int st = kt % STAGES;
    const int k0 = kt * kBK;
    const uint32_t base = lds_base + st * TILE_BYTES;
    if constexpr (S_W > 0) load_scales(kt);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int seg = wave * LOADS + i;
      const uint32_t vo = (k0 + kchunk[i] < p.K) ? voff[i] : kOOB;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(base + seg * 1024);
      dma16(seg < SEG_A ? ra : rb, dst, vo, (uint32_t)k0);
    }
  };

  // fragment: two 16-byte chunks of tile row `row` (lane group g: chunks g and 4 + g)
  auto frag = [&](const uint8_t* base, int row, int sw) -> v8i {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * kBK + ((lg ^ sw) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * kBK + (((4 + lg) ^ sw) << 4));
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
  };

  // Row of the wave's B tile that lane row lr loads for sub-tile j: lane group
  // g' = lr / 4 of the C^T result covers columns [g' * CPL, (g' + 1) * CPL).
  constexpr int CPL = 4 * NT;  // consecutive C columns per lane
  auto brow = [&](int j) { return (lr >> 2) * CPL + 4 * j + (lr & 3); };

  v4f acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- one K step, split into reading its operands (LDS -> registers) and
  // computing on them, so that the two can run in different phases
  v8i fa[MT], fb[NT];
  float bsa[kBlock ? MT : 1];         // block recipes: A row scales (x the B tile scale)
  float bsb[kBlock ? NT : 1][4];      // block 1x128 B: per-column scales
  const uint8_t* la_cur = smem;  // A tile of the step being computed
  auto load_fa = [&](int i) {
    const int row = wm * WM + i * 16 + lr;
    fa[i] = frag(la_cur, row, swz_a(row));
  };
  auto load_step = [&](int kt) {
    const int st = kt % STAGES;
    const uint8_t* la = smem + st * TILE_BYTES;
    const uint8_t* lb = la + BM * kBK;
    la_cur = la;  // A fragments are read in compute(), one M sub-tile ahead of use
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int row = wn * WN + brow(j);
      fb[j] = frag(lb, row, swz_b(row));
    }
    if constexpr (kBlock) {
      if constexpr (REC == kGemmBlock2d) {
        static_assert(WM <= 128 && 128 % WM == 0, "a wave's rows lie inside one 128-row A tile");
        const float sav = __builtin_bit_cast(float, sscale[st][(wm * WM) / 128]);
#pragma unroll
        for (int i = 0; i < MT; ++i) bsa[i] = sav;
      } else {
#pragma unroll
        for (int i = 0; i < MT; ++i) bsa[i] = __builtin_bit_cast(float, sscale[st][wm * WM + i * 16 + lr]);
      }
      if constexpr (kTileB) {
        static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns lie inside one 128-wide B tile");
        const float sbv = __builtin_bit_cast(float, sscale[st][SA_W + (wn * WN) / 128]);
#pragma unroll
        for (int i = 0; i < MT; ++i) bsa[i] *= sbv;
      } else {
        // B scales of this lane's 4 NT columns (lg*CPL .. +CPL), 4 per sub-tile
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const uint4 w = *reinterpret_cast<const uint4*>(&sscale[st][SA_W + wn * WN + lg * CPL + 4 * j]);
          bsb[j][0] = __builtin_bit_cast(float, w.x);
          bsb[j][1] = __builtin_bit_cast(float, w.y);
          bsb[j][2] = __builtin_bit_cast(float, w.z);
          bsb[j][3] = __builtin_bit_cast(float, w.w);
        }
      }
    }
  };
  // The MFMA computes C^T tiles (B fragment first): lane (lr, lg) then holds
  // row i*16 + lr and columns lg*CPL + 4j + r of the wave tile.
  auto compute = [&]() {
    if constexpr (REC == kGemmTensor || REC == kGemmBf16 || REC == kGemmChannel) {
      // A fragment i + 1 is read while sub-tile row i computes; one
      // scheduling region per row keeps two A fragments live
      load_fa(0);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i + 1 < MT) load_fa(i + 1);
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = (REC == kGemmBf16) ? mfma_bf16(fb[j], fa[i], acc[i][j]) : mfma<FB, FA>(fb[j], fa[i], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (kBlock) {
      // Software pipeline: each 128-deep block product goes to a zeroed
      // partial, and the promotion acc += s * partial of sub-tile k - LAG is
      // issued right after the MFMA of sub-tile k, so the FMAs run while the
      // matrix core works (a ring of LAG + 1 partials; the scheduling barriers
      // keep the compiler from regrouping all MFMAs ahead of all FMAs).  A
      // fragments are read one M sub-tile ahead, so two are live at a time.
      constexpr int NSUB = MT * NT, LAG = 4;
      v4f part[LAG + 1];
      load_fa(0);
#pragma unroll
      for (int k = 0; k < NSUB + LAG; ++k) {
        if (k < NSUB && k % NT == 0 && k / NT + 1 < MT) load_fa(k / NT + 1);
        if (k < NSUB) part[k % (LAG + 1)] = mfma<FB, FA>(fb[k % NT], fa[k / NT], v4f{0.0f, 0.0f, 0.0f, 0.0f});
        if (k >= LAG) {
          const int q = k - LAG, i = q / NT, j = q % NT;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sc = kTileB ? bsa[i] : bsa[i] * bsb[j][r];
            acc[i][j][r] = __builtin_fmaf(part[q % (LAG + 1)][r], sc, acc[i][j][r]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // prologue: STAGES - 1 steps in flight
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) {
      issue(s);
      if constexpr (S_W > 0) store_scales(s);
    }

  for (int kt = 0; kt < KT; ++kt) {
    // this step's DMA done (later steps may still be in flight), then make
    // every wave's data visible and retire the stage of step kt - 1
    if (kt + STAGES - 2 < KT)
      wait_vmcnt<LOADS * (STAGES - 2)>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1);

    const int st = kt % STAGES;
    if constexpr (REC == kGemmMx) {
      const uint8_t* la = smem + st * TILE_BYTES;
      const uint8_t* lb = la + BM * kBK;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int row = wn * WN + brow(j);
        fb[j] = frag(lb, row, swz_b(row));
      }
      // lane group lg supplies K block lg: its MT A bytes and NT B bytes
      static_assert(MT % 4 == 0 && NT % 4 == 0, "whole scale words per lane");
      uint32_t sa[MT / 4], sb[NT / 4];
      const uint8_t* sbase = sbytes[st];
#pragma unroll
      for (int q = 0; q < MT / 4; ++q)
        sa[q] = *reinterpret_cast<const uint32_t*>(sbase + lg * BM + wm * WM + lr * MT + 4 * q);
#pragma unroll
      for (int q = 0; q < NT / 4; ++q)
        sb[q] = *reinterpret_cast<const uint32_t*>(sbase + 4 * BM + lg * BN + wn * WN + lr * NT + 4 * q);
      auto load_fa_mx = [&](int i) {
        if (i < 0) return;
        const int row = wm * WM + i * 16 + lr;
        fa[i] = frag(la, row, swz_a(row));
      };
      load_fa_mx(0);
      mx_rows<FA, FB, MT, NT>(std::make_integer_sequence<int, MT>{}, load_fa_mx, acc, fa, fb, sa, sb);
    } else {
      load_step(kt);
      compute();
    }
    // (stored unconditionally: after the last step the stage written is one
    // no wave reads before the next tile refills it)
    if constexpr (S_W > 0) store_scales(kt + STAGES - 1);
  }

  // ---- epilogue: each lane writes CPL consecutive columns of its rows with
  // 16-byte stores (element stores at the matrix edge or for unaligned C)
  float alpha = 1.0f;
  if constexpr (REC == kGemmTensor) {
    if (KT > 0) alpha = *reinterpret_cast<const float*>(p.sa) * *reinterpret_cast<const float*>(p.sb);
  }
  constexpr int ESIZE = OUT == kOutBf16 ? 2 : 4;
  const bool vec_ok = ((p.ldc * ESIZE) % 16 == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
  const int cbase = n0 + wn * WN + lg * CPL;
  // channel scaling: s_b of this lane's CPL columns, s_a per row below
  float csb[REC == kGemmChannel ? CPL : 1];
  if constexpr (REC == kGemmChannel) {
    const float* sb = reinterpret_cast<const float*>(p.sb);
#pragma unroll
    for (int c = 0; c < CPL; ++c) csb[c] = (KT > 0 && cbase + c < p.N) ? sb[cbase + c] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = m0 + wm * WM + i * 16 + lr;
    if (row >= p.M) continue;
    float v[CPL];
    if constexpr (REC == kGemmChannel) {
      const float sar = KT > 0 ? reinterpret_cast<const float*>(p.sa)[row] : 0.0f;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[4 * j + r] = acc[i][j][r] * (sar * csb[4 * j + r]);
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[4 * j + r] = (REC == kGemmTensor) ? acc[i][j][r] * alpha : acc[i][j][r];
    }
    if constexpr (OUT == kOutBf16) {
      __bf16* dst = reinterpret_cast<__bf16*>(p.c) + (int64_t)row * p.ldc + cbase;
      if (vec_ok && cbase + CPL <= p.N) {
#pragma unroll
        for (int q = 0; q < CPL / 8; ++q) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const __bf16 lo = (__bf16)v[8 * q + 2 * e], hi = (__bf16)v[8 * q + 2 * e + 1];
            w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          reinterpret_cast<uint4*>(dst)[q] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          if (cbase + c < p.N) dst[c] = (__bf16)v[c];
      }
    } else {
      float* dst = reinterpret_cast<float*>(p.c) + (int64_t)row * p.ldc + cbase;
      if (vec_ok && cbase + CPL <= p.N) {
#pragma unroll
        for (int q = 0; q < CPL / 4; ++q)
          reinterpret_cast<float4*>(dst)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          if (cbase + c < p.N) dst[c] = v[c];
      }
    }
  }
  }  // tile loop
}

template <int FA, int FB, int REC, int OUT>
hipError_t launch4(const GemmParams& g, hipStream_t st) {
  using C = TileCfg<REC>;
  constexpr int BM = C::BM, BN = C::BN, WAVES_M = C::WAVES_M, WAVES_N = C::WAVES_N;
  // two stages: the scale loads of the block / MX recipes are waited on at
  // the end of each step, which retires that step's tile DMAs as well
  constexpr int STAGES = 2;
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
  // persistent grid: one workgroup per compute unit (the LDS ring admits one)
  const unsigned tiles = (unsigned)a.tiles_m * (unsigned)a.tiles_n;
  const unsigned cus = (unsigned)cu_count(stream_device(st));
  const unsigned blocks = tiles < cus ? tiles : cus;
  gemm_kernel<FA, FB, REC, OUT, BM, BN, WAVES_M, WAVES_N, STAGES>
      <<<blocks, 64 * WAVES_M * WAVES_N, 0, st>>>(a);
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
    case kGemmBlock2d:
      return bf ? launch4<FA, FB, kGemmBlock2d, kOutBf16>(g, st) : launch4<FA, FB, kGemmBlock2d, kOutFp32>(g, st);
    case kGemmChannel:
      return bf ? launch4<FA, FB, kGemmChannel, kOutBf16>(g, st) : launch4<FA, FB, kGemmChannel, kOutFp32>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& g, hipStream_t st) {
  // BF16 operands through the byte-addressed kernel: K and the leading
  // dimensions in bytes, no scales
  GemmParams b = g;
  b.K = 2 * g.K;
  b.lda = 2 * g.lda;
  b.ldb = 2 * g.ldb;
  return g.c_dtype == kOutBf16 ? launch4<kE4M3, kE4M3, kGemmBf16, kOutBf16>(b, st)
                               : launch4<kE4M3, kE4M3, kGemmBf16, kOutFp32>(b, st);
}

hipError_t launch_gemm(const GemmParams& g, hipStream_t st) {
  if (g.fmt_a == kE4M3)
    return g.fmt_b == kE4M3 ? launch_fmt<kE4M3, kE4M3>(g, st) : launch_fmt<kE4M3, kE5M2>(g, st);
  return g.fmt_b == kE4M3 ? launch_fmt<kE5M2, kE4M3>(g, st) : launch_fmt<kE5M2, kE5M2>(g, st);
}

}  // namespace fp8mi
