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
// block-scaled form for MX.  Operand layout of one 16 x 128 fragment: lane l
// holds row l % 16; lane group g = l / 16 holds K bytes [16g, 16g+16) in its
// first four VGPRs and [64+16g, 64+16g+16) in the last four; K block g (bytes
// [32g, 32g+32)) takes its E8M0 scale from lane group g.  Result: lane l,
// register r holds C[4(l/16) + r][l % 16].  The kernel computes C^T
// sub-tiles (B fragment first) with B rows permuted so that each lane owns 16
// consecutive output columns, for 16-byte stores.
//
// Work split: a workgroup of 8 waves computes a 256 x 256 output tile; waves
// 0-3 (group 0) own its rows 0..127, waves 4-7 (group 1) rows 128..255, and
// wave q of a group columns 64q..64q+63 (a 128 x 64 sub-tile, 8 x 4 MFMA
// products per 128-deep K step).  Operand tiles stream HBM -> LDS with
// buffer_load ... lds (no VGPR staging) into two 64 KB stages, each row's
// 16-byte chunks XOR-swizzled so fragment reads hit distinct banks; rows past
// the matrix and K past its end come back as zeros from the buffer's range
// check.
//
// Schedule ("ping-pong"): a K step k is two phases with a workgroup barrier
// after each.  In phase 2k group 0 reads its B fragments of step k from LDS
// and issues DMA while group 1 multiplies step k-1; in phase 2k+1 group 0
// multiplies step k (streaming its A fragments from LDS one 16-row sub-tile
// ahead of the products) while group 1 reads and issues.  So on every SIMD
// one wave feeds the matrix core while the other reads LDS and moves data,
// instead of both waiting on the same barrier and reading at the same time.
// DMA duty: in its load phase of step k each group brings its own half of
// the A tile of step k+1 (and those rows' scales), group 0 also the B tile;
// each lands in the stage step k-1 left, and every wave waits for its own set
// at the end of its multiply phase.  A group's A half is therefore readable
// in its own next load phase, which preloads the first A sub-tile (and the
// MX row bytes) so that the multiply phase opens with MFMAs.
//
// Scale application:
//   TENSOR      one alpha = s_a * s_b on the FP32 accumulator at the end;
//   CHANNEL     s_a[row] * s_b[col] on the FP32 accumulator at the end;
//   MX          E8M0 scales fed to the scaled MFMA (no VALU work);
//   BLOCK_*     each 128-deep K block is an MFMA into a zeroed FP32 partial,
//               then acc += (s_a[row, kb] * s_b[.., kb]) * partial on the VALU,
//               four products behind the matrix core; the last row's
//               promotions of a step run at the start of the wave's next
//               load phase, off the matrix core's critical path.
// Scale words travel like the tiles, by LDS DMA, but four K steps at a time:
// one 16-byte request per operand row brings the row's scales of four steps
// (a per-step dword would cost the texture path one cache-line request per
// row per step), into two small group buffers beside the tile stages.
//
// The same kernel, with BF16 operands and v_mfma_f32_16x16x32_bf16, is the
// BF16 GEMM FP8's speedup is measured against ("Mastering FP8 LLM training",
// Fig. 1): a 128-byte K step is 64 BF16 elements, the two 16-byte halves of a
// fragment feed two 32-deep products, and everything else is shared.
#include <utility>

#include "device.hpp"
#include "launch.hpp"

namespace fp8mi {

namespace {

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>): indices into
// register arrays stay compile-time constants whatever the unroller decides
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 128;                 // K bytes per step
constexpr uint32_t kOOB = 0x80000000u;   // voffset past every buffer's range
constexpr int kBM = 256, kBN = 256;      // workgroup tile
constexpr int kWM = 128, kWN = 64;       // wave tile
constexpr int kMT = kWM / 16, kNT = kWN / 16;
constexpr int kCPL = 4 * kNT;            // consecutive C columns per lane
constexpr int kTileBytes = (kBM + kBN) * kBK;
constexpr int kLag = 4;                  // promotion distance behind the MFMAs
constexpr int kAhead = 1;                // A sub-tiles read ahead of the MFMAs
constexpr int kRingA = kAhead + 1;       // A fragments held
constexpr int kRingS = kAhead + 2;       // A row scales held (a row's promotions trail one row)
// Scales travel in groups of kSG K steps, two group buffers: each operand
// row's FP32 words (or E8M0 bytes) for the group as 16 bytes at LO + 16 row,
// taken from the aligned dword holding the first; an MX row whose bytes run
// past those 16 takes the dword after them from HI + 4 row.  A 128-row tile
// scale takes 16 bytes per tile at LO + 1024 t (A) or LO + 16 t (B).
constexpr int kSG = 4;
constexpr int kSclALo = 0, kSclAHi = 4096, kSclBLo = 5120, kSclBHi = 9216, kSclBytes = 10240;

template <int FA, int FB>
__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz / blgp select the operand formats: 0 = E4M3, 1 = E5M2
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// E8M0 scales in byte 0 of each scale register
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

// BF16 operands: the 32-byte fragment holds K elements [8g, 8g+8) and
// [32+8g, 32+8g+8) of lane group g; A and B use the same lane -> K map, so
// two 32-deep products cover the 64-deep step.
__device__ __forceinline__ v4f mfma_bf16(const v8i& a, const v8i& b, v4f c) {
  const v4i a0 = {a[0], a[1], a[2], a[3]}, a1 = {a[4], a[5], a[6], a[7]};
  const v4i b0 = {b[0], b[1], b[2], b[3]}, b1 = {b[4], b[5], b[6], b[7]};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v8bf, b0), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v8bf, b1), c, 0, 0, 0);
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

// 16 bytes of LDS at byte address addr (a constant added to addr lands in the
// instruction's offset field)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_u4(uint32_t addr) {
  const u32x4_t v = *(__attribute__((address_space(3))) const u32x4_t*)(size_t)addr;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float lds_f32(uint32_t addr) {
  return *(__attribute__((address_space(3))) const float*)(size_t)addr;
}
__device__ __forceinline__ int lds_u8(uint32_t addr) {
  return *(__attribute__((address_space(3))) const uint8_t*)(size_t)addr;
}

// Wave-wide LDS DMA: LDS[m0 + 16 * lane] (dwordx4) or LDS[m0 + 4 * lane]
// (dword) = buffer[voff + soff].  Inline asm so that the compiler's wait-count
// pass does not treat it as an LDS store aliasing every later LDS read (which
// would drain vmcnt before each fragment read); completion is tracked with
// wait_vmcnt.  The s_nop covers the M0-write -> LDS-DMA wait state.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// s_waitcnt vmcnt(n) / lgkmcnt(0), the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

struct GArgs {
  const uint8_t* a;
  const uint8_t* b;
  const void* sa;
  const void* sb;
  int64_t lda, ldb, ldc;
  int M, N, K;
  int nkb;  // scale entries per operand row: K blocks of 128 (FP32 words) or of 32 (MX bytes)
  void* c;
  int tiles_m, tiles_n;
};

// What each recipe stages per K step.
template <int REC>
struct Scl {
  static constexpr bool kRowA = REC == kGemmBlock128x128 || REC == kGemmBlock1x128;  // FP32 per A row
  static constexpr bool kTileA = REC == kGemmBlock2d;                                 // FP32 per 128-row A tile
  static constexpr bool kRowB = REC == kGemmBlock1x128;                               // FP32 per B row
  static constexpr bool kTileB = REC == kGemmBlock128x128 || REC == kGemmBlock2d;     // FP32 per 128-row B tile
  static constexpr bool kMx = REC == kGemmMx;
  static constexpr bool kPromote = kRowA || kTileA;
  static constexpr bool kSclAny = kRowA || kTileA || kRowB || kTileB || kMx;
  // the wave's 12 DMA source offsets held in registers for the whole kernel
  // (the channel, per-B-row-scale, MX and 1x128 x 128x128 kernels have no
  // room for them)
  static constexpr bool kHoistDma = !kRowB && !kMx && REC != kGemmChannel && REC != kGemmBlock128x128;
};

template <int FA, int FB, int REC, int OUT>
__global__ __launch_bounds__(512, 1) void gemm_kernel(GArgs p) {
  using S = Scl<REC>;
  constexpr bool kScl = S::kSclAny;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sscl[2][kScl ? kSclBytes : 16];

  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)smem;
  const uint32_t scl_base = (uint32_t)(uintptr_t)(lds_void*)&sscl[0][0];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int grp = wave >> 2, q = wave & 3;
  const int wm = grp, wn = q;
  const int lr = lane & 15;  // fragment row
  const int lg = lane >> 4;  // lane group
  // LDS byte offsets (within a stage) of the two 16-byte halves of the first
  // fragment row this lane reads: A row wm kWM + lr, B row wn kWN + (lr / 4)
  // CPL + lr % 4.  Its later rows (A: + 16 per sub-tile, B: + 4 per
  // sub-tile, bits 0, 1 and 4 of the row unchanged) share that row's
  // swizzle, so every fragment read is one of these plus a constant.
  const int arow = wm * kWM + lr, brow0 = wn * kWN + (lr >> 2) * kCPL + (lr & 3);
  const int swa = swz_a(arow), swb = swz_b(brow0);
  const uint32_t fa_lo = (uint32_t)(arow * kBK + ((lg ^ swa) << 4));
  const uint32_t fa_hi = (uint32_t)(arow * kBK + (((4 + lg) ^ swa) << 4));
  const uint32_t fb_lo = (uint32_t)(kBM * kBK + brow0 * kBK + ((lg ^ swb) << 4));
  const uint32_t fb_hi = (uint32_t)(kBM * kBK + brow0 * kBK + (((4 + lg) ^ swb) << 4));


  const int total = p.tiles_m * p.tiles_n;
#pragma unroll 1
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    __syncthreads();  // every wave is done with the previous tile's LDS
    // ---- tile assignment: XCD-contiguous ranges of the tile index (tiles t and
    // t + gridDim.x stay on one XCD when gridDim.x % 8 == 0), grouped 8 tile-rows deep
    int pid = tile;
    if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
    constexpr int GROUP_M = 8;
    const int in_group = GROUP_M * p.tiles_n;
    const int first_m = (pid / in_group) * GROUP_M;
    const int gsize = min(p.tiles_m - first_m, GROUP_M);
    const int pm = first_m + (pid % in_group) % gsize;
    const int pn = (pid % in_group) / gsize;
    const int m0 = pm * kBM, n0 = pn * kBN;
    const int rows_a = min(kBM, p.M - m0), rows_b = min(kBN, p.N - n0);
    const int KT = (p.K + kBK - 1) / kBK;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.lda, (uint32_t)(rows_a * p.lda));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (int64_t)n0 * p.ldb, (uint32_t)(rows_b * p.ldb));
    // scale rows of this tile (range-checked: rows past the matrix read as zero)
    __amdgpu_buffer_rsrc_t rsa = make_rsrc(nullptr, 0), rsb = make_rsrc(nullptr, 0);
    if constexpr (S::kRowA)
      rsa = make_rsrc(static_cast<const uint32_t*>(p.sa) + (int64_t)m0 * p.nkb, (uint32_t)(rows_a * p.nkb * 4));
    if constexpr (S::kTileA)
      rsa = make_rsrc(static_cast<const uint32_t*>(p.sa) + (int64_t)(m0 / 128) * p.nkb,
                      (uint32_t)(((rows_a + 127) / 128) * p.nkb * 4));
    if constexpr (S::kMx)
      rsa = make_rsrc(static_cast<const uint8_t*>(p.sa) + (int64_t)m0 * p.nkb, (uint32_t)((rows_a * p.nkb + 3) & ~3));
    if constexpr (S::kRowB)
      rsb = make_rsrc(static_cast<const uint32_t*>(p.sb) + (int64_t)n0 * p.nkb, (uint32_t)(rows_b * p.nkb * 4));
    if constexpr (S::kTileB)
      rsb = make_rsrc(static_cast<const uint32_t*>(p.sb) + (int64_t)(n0 / 128) * p.nkb,
                      (uint32_t)(((rows_b + 127) / 128) * p.nkb * 4));
    if constexpr (S::kMx)
      rsb = make_rsrc(static_cast<const uint8_t*>(p.sb) + (int64_t)n0 * p.nkb, (uint32_t)((rows_b * p.nkb + 3) & ~3));

    // One 1 KB tile segment (8 rows): segments 0..31 are A rows 8s.., 32..63
    // B rows 8(s-32)...  Lane l fetches chunk (l % 8) ^ swizzle of row 8s + l / 8: for an A row
    // the swizzle is l / 8 whatever s is, for a B row (l / 8) % 4 plus 4 x
    // bit 1 of s (see swz_b); so a lane's source offset is one of three
    // per-lane bases plus the wave-uniform 8 s ld.  The K-tail check (chunks
    // past K read as zeros) runs only in the step that has one.
    auto chunk = [&](bool is_a, int seg) __attribute__((always_inline)) -> int {
      return 16 * ((lane & 7) ^ (is_a ? (lane >> 3) : (((lane >> 3) & 3) | ((seg & 2) << 1))));
    };
    const uint32_t base_a = (uint32_t)((lane >> 3) * p.lda + chunk(true, 0));
    const uint32_t base_b0 = (uint32_t)((lane >> 3) * p.ldb + chunk(false, 0));
    const uint32_t base_b1 = (uint32_t)((lane >> 3) * p.ldb + chunk(false, 2));
    // this wave's segments' offsets: A 16 grp + 4 q + i, B 32 + 8 q + i
    uint32_t voa[S::kHoistDma ? 4 : 1], vob[S::kHoistDma ? 8 : 1];
    if constexpr (S::kHoistDma) {
#pragma unroll
      for (int i = 0; i < 4; ++i) voa[i] = base_a + (uint32_t)(8 * (16 * grp + 4 * q + i)) * (uint32_t)p.lda;
#pragma unroll
      for (int i = 0; i < 8; ++i) vob[i] = ((i & 2) ? base_b1 : base_b0) + (uint32_t)(8 * (8 * q + i)) * (uint32_t)p.ldb;
    }
    // (is_a is a constant at each call; the operand's resource and row stride
    // come in by value: a pick between the two variables would take their
    // addresses and keep them in private memory)
    auto dma_tile = [&](int seg, int kt, bool is_a, __amdgpu_buffer_rsrc_t rs, int stride, auto Tail, int i)
        __attribute__((always_inline)) {
      const int k0 = kt * kBK;
      // the segment's offset: from the registers set above, or the lane's
      // base plus the wave-uniform row offset 8 s ld (formed on the scalar
      // unit; ld passes through an empty asm so that it is formed at each
      // use, not hoisted per segment).  Either way the row part sits in the
      // range-checked vector offset, so rows past the matrix read as zero.
      uint32_t vo;
      if constexpr (S::kHoistDma) {
        vo = is_a ? voa[i] : vob[i];
      } else {
        uint32_t ld = __builtin_amdgcn_readfirstlane((uint32_t)stride);
        asm volatile("" : "+s"(ld));
        vo = (is_a ? base_a : ((seg & 2) ? base_b1 : base_b0)) + (uint32_t)(8 * (seg & 31)) * ld;
      }
      if constexpr (decltype(Tail)::value) {
        if (k0 + chunk(is_a, seg) >= p.K) vo = kOOB;
      }
      uint32_t lb = __builtin_amdgcn_readfirstlane(lds_base + (kt & 1) * kTileBytes);
      asm volatile("" : "+s"(lb));
      dma16(rs, lb + seg * 1024, vo, (uint32_t)k0);
    };
    // Scales of the kSG steps from kt on (kt a multiple of kSG) into group
    // buffer (kt / kSG) & 1.  A side, each group its own 128 rows: waves
    // q = 0, 1 bring rows 128 g + 64 q + l (16 bytes each), MX waves q = 2, 3
    // the dwords after them; a 128-row tile scale comes from lane 0 of wave
    // 0.  B side, group 0: wave q brings rows 64 q + l (MX: and the dwords
    // after them), or lanes 0 and 1 of wave 0 the two tiles' words.  Lanes
    // with nothing to bring read past the range (zeros) into slack space.
    auto dma_scl = [&](int kt, bool a_side, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
      uint32_t sb = __builtin_amdgcn_readfirstlane(scl_base + ((kt / kSG) & 1) * kSclBytes);
      asm volatile("" : "+s"(sb));
      auto first = [&](int row) -> uint32_t {  // aligned start of a row's group window
        return S::kMx ? ((((uint32_t)(row * p.nkb)) & ~3u) + 4u * kt) : (uint32_t)((row * p.nkb + kt) * 4);
      };
      if (a_side) {
        if constexpr (S::kTileA) {
          if (q == 0) dma16(rs, sb + kSclALo + 1024 * grp, lane == 0 ? (uint32_t)((grp * p.nkb + kt) * 4) : kOOB, 0);
        } else {
          if (q < 2) dma16(rs, sb + kSclALo + 16 * (128 * grp + 64 * q), first(128 * grp + 64 * q + lane), 0);
          if constexpr (S::kMx)
            if (q >= 2) dma4(rs, sb + kSclAHi + 4 * (128 * grp + 64 * (q - 2)), first(128 * grp + 64 * (q - 2) + lane) + 16u);
        }
      } else {
        if constexpr (S::kTileB) {
          if (q == 0) dma16(rs, sb + kSclBLo, lane < 2 ? (uint32_t)((lane * p.nkb + kt) * 4) : kOOB, 0);
        } else {
          dma16(rs, sb + kSclBLo + 16 * 64 * q, first(64 * q + lane), 0);
          if constexpr (S::kMx) dma4(rs, sb + kSclBHi + 4 * 64 * q, first(64 * q + lane) + 16u);
        }
      }
    };
    // This wave's DMA set for step kt.  Each group moves its own 128 A rows
    // (wave q: segments 4 q.. of its half) and their scales; group 0 also
    // the whole B tile (wave q: segments 32 + 8 q..) and B scales.  Scales
    // go out with the first step of each group of kSG.
    auto issue_set = [&](int kt, auto Tail) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma_tile(16 * grp + 4 * q + i, kt, true, ra, p.lda, Tail, i);
      const bool scl = (kt % kSG) == 0;
      if constexpr (S::kRowA || S::kTileA || S::kMx)
        if (scl) dma_scl(kt, true, rsa);
      if (grp == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dma_tile(32 + 8 * q + i, kt, false, rb, p.ldb, Tail, i);
        if constexpr (S::kRowB || S::kTileB || S::kMx)
          if (scl) dma_scl(kt, false, rsb);
      }
    };
    auto issue = [&](int kt) __attribute__((always_inline)) {
      if (kt * kBK + kBK <= p.K) issue_set(kt, std::false_type{});
      else issue_set(kt, std::true_type{});
    };

    // ---- registers
    v4f acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
      for (int j = 0; j < kNT; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    v8i fa[kRingA], fb[kNT];
    // (zero-initialised: the tail promotion at the top of step 0 then adds
    // 0 * 0, so it runs unconditionally -- a conditional update of acc would
    // make the compiler copy all 128 accumulators at the branch's merge)
    v4f part[kLag + 1];                          // block partials, a ring
    float bsa[S::kRowA ? kRingS : 1];            // A row scales of rows i-1 .. i+kAhead, a ring
    float bsb[S::kRowB ? kNT : 1][4];            // B column scales of the lane's columns
    float stile = 0.0f;                          // B tile scale (x A tile scale for 2-D)
#pragma unroll
    for (int t = 0; t < kLag + 1; ++t) part[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < (S::kRowA ? kRingS : 1); ++t) bsa[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < (S::kRowB ? kNT : 1); ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) bsb[j][r] = 0.0f;
    int sax[S::kMx ? kMT : 1], sbx[S::kMx ? kNT : 1];  // E8M0 bytes of the lane's rows / columns

    // per-step LDS addresses of the lane's fragment rows (stage kt & 1) and
    // of its A row scales, formed once per step in the load phase; every
    // sub-tile's read then adds only a constant.  The empty asm keeps each a
    // single register value, so the compiler does not re-form it per read.
    uint32_t sa_lo = 0, sa_hi = 0, sb_lo = 0, sb_hi = 0, ssa = 0;
    auto frag = [&](uint32_t lo_addr, uint32_t hi_addr) __attribute__((always_inline)) -> v8i {
      const uint4 lo = lds_u4(lo_addr);
      const uint4 hi = lds_u4(hi_addr);
      v8i f;
      f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
      f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
      return f;
    };
    // B row (tile row within the wave's 64) that lane row lr loads for sub-tile j:
    // lane group g' = lr / 4 of the C^T result covers columns [g' CPL, (g'+1) CPL)
    auto brow = [&](int j) __attribute__((always_inline)) { return (lr >> 2) * kCPL + 4 * j + (lr & 3); };
    // MX: lane group lg feeds K block 4 kt + lg of its row.  A row's bytes
    // for a scale group start mis = (row nkb) % 4 bytes into its staged
    // window (16 bytes from the aligned dword holding the first, then the
    // dword after them); mis is ((lr % 4) nkb) % 4 for every row a lane reads
    // (tiles start on multiples of 4 rows), so the lane's byte of step kt is
    // window byte b = mis + lg + 4 (kt % kSG), the same for all its rows.
    auto mx_b = [&](int kt) __attribute__((always_inline)) -> int {
      return (((lr & 3) * p.nkb) & 3) + lg + 4 * (kt % kSG);
    };
    // where row `row`'s byte b sits: in its 16 bytes at LO, or in the dword after at HI
    auto mx_at = [&](const uint8_t* sc, int lo, int hi, int row, int b) __attribute__((always_inline)) -> const uint8_t* {
      return b < 16 ? sc + lo + 16 * row + b : sc + hi + 4 * row + (b - 16);
    };
    // E8M0 byte of a row (in the last step, blocks past K are masked at the
    // start of the multiply phase)
    auto mx_byte = [&](const uint8_t* at) __attribute__((always_inline)) -> int { return *at; };

    // promotion of product t = i * NT + j: acc[i][j] += s * part
    auto promote = [&](auto T) __attribute__((always_inline)) {
      if constexpr (S::kPromote) {
        constexpr int t = decltype(T)::value;
        constexpr int i = t / kNT, j = t % kNT;
        static_for<4>([&](auto R) {
          constexpr int r = decltype(R)::value;
          float sc;
          if constexpr (S::kRowB) sc = bsa[i % kRingS] * bsb[j][r];
          else if constexpr (S::kRowA) sc = bsa[i % kRingS] * stile;
          else sc = stile;
          acc[i][j][r] = __builtin_fmaf(part[t % (kLag + 1)][r], sc, acc[i][j][r]);
        });
        // pin the update here: left to itself the compiler sinks every
        // promotion of a phase past the barrier, keeping 32 partials alive
        asm volatile("" : "+v"(acc[i][j]));
      }
    };

    // A sub-tile i of the step whose addresses the load phase set (rows 16 i..
    // of the group's half) and its row scale
    auto load_a = [&](int i) __attribute__((always_inline)) {  // i is a constant at every (inlined) call
      fa[i % kRingA] = frag(sa_lo + (uint32_t)(i * 16 * kBK), sa_hi + (uint32_t)(i * 16 * kBK));
      if constexpr (S::kRowA) bsa[i % kRingS] = lds_f32(ssa + (uint32_t)(16 * 16 * i));
    };

    // ---- load phase of step kt: B fragments and B-side scales into
    // registers, then the first A sub-tile of the group's own half
    auto load_phase = [&](int kt) __attribute__((always_inline)) {
      const uint32_t stage = lds_base + (uint32_t)((kt & 1) * kTileBytes);
      sa_lo = fa_lo + stage;
      sa_hi = fa_hi + stage;
      sb_lo = fb_lo + stage;
      sb_hi = fb_hi + stage;
      if constexpr (S::kRowA)
        ssa = scl_base + (uint32_t)(((kt / kSG) & 1) * kSclBytes + kSclALo + 16 * arow + 4 * (kt % kSG));
      asm volatile("" : "+v"(sa_lo), "+v"(sa_hi), "+v"(sb_lo), "+v"(sb_hi));
      if constexpr (S::kRowA) asm volatile("" : "+v"(ssa));
#pragma unroll
      for (int j = 0; j < kNT; ++j) fb[j] = frag(sb_lo + (uint32_t)(4 * j * kBK), sb_hi + (uint32_t)(4 * j * kBK));
      const uint8_t* sc = &sscl[(kt / kSG) & 1][0];
      const int ks = 4 * (kt % kSG);  // the step's word in a row's 16 bytes
      if constexpr (S::kRowB) {
        uint32_t ssb = scl_base + (uint32_t)(((kt / kSG) & 1) * kSclBytes + kSclBLo + 16 * (wn * kWN + lg * kCPL) + ks);
        asm volatile("" : "+v"(ssb));
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            bsb[j][e] = lds_f32(ssb + (uint32_t)(16 * (4 * j + e)));
      }
      if constexpr (S::kTileB) stile = *reinterpret_cast<const float*>(sc + kSclBLo + 16 * (wn / 2) + ks);
      // this group's own A rows (landed by its own waits): the 2-D recipe's
      // A tile scale, the MX row bytes, and the first sub-tile, so that the
      // multiply phase opens with MFMAs
      if constexpr (S::kTileA) stile *= *reinterpret_cast<const float*>(sc + kSclALo + 1024 * wm + ks);
      if constexpr (S::kMx) {
        const int b = mx_b(kt);
        if (kt % kSG < kSG - 1) {
          // b <= 14: every lane's byte is among its rows' 16 staged bytes,
          // at a constant distance from its first row's
          uint32_t xa = scl_base + (uint32_t)(((kt / kSG) & 1) * kSclBytes + kSclALo + 16 * arow + b);
          uint32_t xb = scl_base + (uint32_t)(((kt / kSG) & 1) * kSclBytes + kSclBLo + 16 * brow0 + b);
          asm volatile("" : "+v"(xa), "+v"(xb));
#pragma unroll
          for (int i = 0; i < kMT; ++i) sax[i] = lds_u8(xa + (uint32_t)(16 * 16 * i));
#pragma unroll
          for (int j = 0; j < kNT; ++j) sbx[j] = lds_u8(xb + (uint32_t)(16 * 4 * j));
        } else {
#pragma unroll
          for (int i = 0; i < kMT; ++i) sax[i] = mx_byte(mx_at(sc, kSclALo, kSclAHi, wm * kWM + i * 16 + lr, b));
#pragma unroll
          for (int j = 0; j < kNT; ++j) sbx[j] = mx_byte(mx_at(sc, kSclBLo, kSclBHi, wn * kWN + brow(j), b));
        }
      }
#pragma unroll
      for (int i = 0; i < kAhead; ++i) load_a(i);
    };

    // ---- multiply phase of step kt: A fragments (and A row scales) stream
    // from LDS one 16-row sub-tile ahead of the products
    auto compute_phase = [&](int kt) __attribute__((always_inline)) {
      // MX: blocks past K (last step only) take byte 0, 2^-127, times their
      // zero codes, whatever E8M0 bytes follow a row's last
      if constexpr (S::kMx) {
        if (p.nkb - 4 * kt < 4) {
          const bool in_k = lg < p.nkb - 4 * kt;
#pragma unroll
          for (int i = 0; i < kMT; ++i) sax[i] = in_k ? sax[i] : 0;
#pragma unroll
          for (int j = 0; j < kNT; ++j) sbx[j] = in_k ? sbx[j] : 0;
        }
      }
      static_for<kMT>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i + kAhead < kMT) load_a(i + kAhead);
        static_for<kNT>([&](auto J) {
          constexpr int j = decltype(J)::value;
          constexpr int t = i * kNT + j;
          if constexpr (S::kPromote) {
            part[t % (kLag + 1)] = mfma<FB, FA>(fb[j], fa[i % kRingA], v4f{0.0f, 0.0f, 0.0f, 0.0f});
            if constexpr (t >= kLag) promote(std::integral_constant<int, t - kLag>{});
            // one scale per product (an A row or tile scale times the B tile
            // scale): each MFMA followed by exactly the four promotion FMAs
            // of the product kLag before it.  The wave's in-order issue hides
            // an even four per 16x16x128 product far better than the uneven
            // groups the scheduler forms by itself
            if constexpr (!S::kRowB) __builtin_amdgcn_sched_barrier(0);
          } else if constexpr (S::kMx) {
            acc[i][j] = mfma_mx<FB, FA>(fb[j], fa[i % kRingA], acc[i][j], sbx[j], sax[i]);
          } else if constexpr (REC == kGemmBf16) {
            acc[i][j] = mfma_bf16(fb[j], fa[i % kRingA], acc[i][j]);
          } else {
            acc[i][j] = mfma<FB, FA>(fb[j], fa[i % kRingA], acc[i][j]);
          }
        });
        // keep the row's products in this phase: the MFMAs are pure, and left
        // to itself the compiler sinks them below the phase's waits and
        // barrier, holding every A fragment of the step live until then
        if constexpr (!S::kPromote)
          asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]), "+v"(acc[i][2]), "+v"(acc[i][3]));
        // per-column B scales as well (a scale product and an FMA per
        // element): each MFMA followed by up to 6 VALU instructions of the
        // promotion arithmetic and one LDS read, so that the wave's in-order
        // issue keeps the matrix pipe fed while the VALU work drains (a row
        // carries 32 of them; groups of 6 timed best, ahead of 3-5, 7-12
        // and a strict eight after each MFMA)
        if constexpr (S::kPromote && S::kRowB) {
          static_for<kNT>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // the last row's promotions, left for the start of the next load phase
    auto promote_tail = [&]() __attribute__((always_inline)) {
      if constexpr (S::kPromote) {
        static_for<kLag>([&](auto T) {
          promote(std::integral_constant<int, kMT * kNT - kLag + decltype(T)::value>{});
        });
      }
    };

    // ---- prologue: steps 0 and 1 whole, each wave its own DMA set of each
    if (0 < KT) issue(0);
    if (1 < KT) issue(1);
    // channel scaling: the lane's row and column scales, fetched now so that
    // a short K loop does not end waiting on them
    const int cbase = n0 + wn * kWN + lg * kCPL;  // first of the lane's CPL output columns
    float csa[REC == kGemmChannel ? kMT : 1], csb[REC == kGemmChannel ? kCPL : 1];
    if constexpr (REC == kGemmChannel) {
      const float* sap = reinterpret_cast<const float*>(p.sa);
      const float* sbp = reinterpret_cast<const float*>(p.sb);
#pragma unroll
      for (int c = 0; c < kCPL; ++c) csb[c] = (KT > 0 && cbase + c < p.N) ? sbp[cbase + c] : 0.0f;
#pragma unroll
      for (int i = 0; i < kMT; ++i) {
        const int row = m0 + wm * kWM + i * 16 + lr;
        csa[i] = (KT > 0 && row < p.M) ? sap[row] : 0.0f;
      }
    }
    wait_vmcnt<0>();
    __syncthreads();

    // Every wave runs L(k); barrier; C(k); barrier for k = 0 .. KT-1; group 1
    // passes one barrier first and group 0 one last, so group 0's L(k) and
    // C(k) fall in phases 2k and 2k+1, group 1's in 2k+1 and 2k+2.  The set
    // for step k+1 goes out in L(k) (step 1 came in the prologue) into the
    // stage step k-1 left: its B was read in L0(k-1) and L1(k-1), each A half
    // (and its scales) by its own group in L(k-1) and C(k-1), all in phases
    // before L0(k) / L1(k).  Each wave waits for its whole set at the end of
    // C(k), so the barrier there publishes group 0's B for L0(k+1) and every
    // group's A half for its own L(k+1).  Scales go out with the first step
    // of each group of kSG into the group buffer last used kSG to 2 kSG - 1
    // steps before, whose last reads are long done.
    if (grp == 1) __syncthreads();
#pragma unroll 1
    for (int k = 0; k < KT; ++k) {
      promote_tail();
      if (k >= 1 && k + 1 < KT) issue(k + 1);
      load_phase(k);
      wait_lgkm0();
      __syncthreads();
      compute_phase(k);
      wait_lgkm0();  // done reading stage k & 1
      wait_vmcnt<0>();
      __syncthreads();
    }
    promote_tail();

    // ---- epilogue: each lane writes CPL consecutive columns of its rows with
    // 16-byte stores (element stores at the matrix edge or for unaligned C);
    // group 0 stores while group 1 finishes its last step
    float alpha = 1.0f;
    if constexpr (REC == kGemmTensor) {
      if (KT > 0) alpha = *reinterpret_cast<const float*>(p.sa) * *reinterpret_cast<const float*>(p.sb);
    }
    constexpr int ESIZE = OUT == kOutBf16 ? 2 : 4;
    const bool vec_ok = ((p.ldc * ESIZE) % 16 == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      const int row = m0 + wm * kWM + i * 16 + lr;
      if (row >= p.M) continue;
      float v[kCPL];
      if constexpr (REC == kGemmChannel) {
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[4 * j + r] = acc[i][j][r] * (csa[i] * csb[4 * j + r]);
      } else {
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[4 * j + r] = (REC == kGemmTensor) ? acc[i][j][r] * alpha : acc[i][j][r];
      }
      if constexpr (OUT == kOutBf16) {
        __bf16* dst = reinterpret_cast<__bf16*>(p.c) + (int64_t)row * p.ldc + cbase;
        if (vec_ok && cbase + kCPL <= p.N) {
#pragma unroll
          for (int qq = 0; qq < kCPL / 8; ++qq) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const __bf16 lo = (__bf16)v[8 * qq + 2 * e], hi = (__bf16)v[8 * qq + 2 * e + 1];
              w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            reinterpret_cast<uint4*>(dst)[qq] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < kCPL; ++c)
            if (cbase + c < p.N) dst[c] = (__bf16)v[c];
        }
      } else {
        float* dst = reinterpret_cast<float*>(p.c) + (int64_t)row * p.ldc + cbase;
        if (vec_ok && cbase + kCPL <= p.N) {
#pragma unroll
          for (int qq = 0; qq < kCPL / 4; ++qq)
            reinterpret_cast<float4*>(dst)[qq] = make_float4(v[4 * qq], v[4 * qq + 1], v[4 * qq + 2], v[4 * qq + 3]);
        } else {
#pragma unroll
          for (int c = 0; c < kCPL; ++c)
            if (cbase + c < p.N) dst[c] = v[c];
        }
      }
    }
    if (grp == 0) __syncthreads();
  }  // tile loop
}

template <int FA, int FB, int REC, int OUT>
hipError_t launch4(const GemmParams& g, hipStream_t st) {
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
  a.nkb = REC == kGemmMx ? (int)((g.K + 31) / 32) : (int)((g.K + 127) / 128);
  a.c = g.c;
  a.tiles_m = (int)((g.M + kBM - 1) / kBM);
  a.tiles_n = (int)((g.N + kBN - 1) / kBN);
  // persistent grid: one workgroup per compute unit (the LDS ring admits one)
  const unsigned tiles = (unsigned)a.tiles_m * (unsigned)a.tiles_n;
  const unsigned cus = (unsigned)cu_count(stream_device(st));
  const unsigned blocks = tiles < cus ? tiles : cus;
  gemm_kernel<FA, FB, REC, OUT><<<blocks, 512, 0, st>>>(a);
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
