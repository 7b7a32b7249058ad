// Weight-only 4-bit GEMM for prefill: C[m][r] = bf16( sum_c A[m][c] * W[r][c] ).
//
// The page names this kernel w4a16_gemm, a weight-only 4-bit GEMM for prefill
// ("Feasibility Report: Porting ROCmFP4 to Atlas", "Kernel System"). Prefill is a
// dense contraction, so it runs on the matrix cores: each workgroup decodes a tile of
// packed weights into LDS as bf16 (exact: every codebook value times every decoded
// scale is a bf16 value) and feeds v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
// the epilogue rounds to bf16 (nearest even).
//
// Tiling. The main configuration is a 512-thread workgroup (8 wavefronts, two per
// SIMD) owning a 256 x 256 tile of C (256 rows of A by 256 weight rows); each
// wavefront computes a 64 x 128 sub-tile as 2 x 4 MFMA tiles of 32 x 32 (128 fp32
// accumulators per lane). Each step consumes 64 columns of K, i.e. two ROCmFP4 blocks
// per weight row.
//
// Balance. A grid of equal tiles runs in whole rounds over the CUs, so 544 tiles on
// 256 CUs would take three rounds for 2.125 rounds of work. The launcher therefore
// computes the last columns of C as 128 x 128 tiles (a 256-thread configuration of four
// wavefronts, one per SIMD, each owning 64 x 64), run by a second launch, and may split
// the k range of either kind of tile; a cost model of the launch picks the plan.
//
// Pipeline (LDS double-buffered, one barrier per step). While step s is multiplied out
// of LDS buffer s % 2:
//   * the A tile of step s+1 is loaded into registers (four 16-byte chunks per thread)
//     and written to the other buffer after the MFMAs;
//   * the packed weights of step s+1 (loaded one step earlier) are decoded to bf16 into
//     the other buffer, one 16-byte chunk per 16-column k slice, interleaved with that
//     slice's MFMAs; the weights of step s+2 are loaded.
// LDS rows are 64 bf16 (eight 16-byte chunks) with the chunk index XOR-swizzled by the
// row, so the MFMA fragment reads (32 consecutive rows, one chunk) hit distinct banks.
//
// Mapping. Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2. The tile order (tile_coords) arranges the XCDs as a grid over (M tiles, N strips)
// chosen to move the fewest bytes of A and W across the fabric: for the prefill shape
// 2 x 4, so each XCD works on 4 row slabs of A and a quarter of the weight strips
// (main-tile fabric reads 265 MB per call, against 430 MB when every XCD streamed all
// of W; the kernel time is the same either way).

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "rfp4_decode.h"
#include "rfp4_internal.h"

namespace rfp4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;

// Weight decode through a per-workgroup table in LDS (1) or with converts and
// multiplies (0); see decode_chunk.
#ifndef RFP4_GEMM_LUT
#define RFP4_GEMM_LUT 1
#endif

// Tile configuration: BM x BN tile of C per workgroup, WM x WN wavefronts.
template <int BM_, int BN_, int WM_, int WN_, int PD_ = 1, bool PP_ = false>
struct TileCfg {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int WM = WM_;
  static constexpr int WN = WN_;
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kWaveM = BM / WM;  // rows of C per wavefront
  static constexpr int kWaveN = BN / WN;  // columns of C per wavefront
  static constexpr int TM = kWaveM / 32;  // MFMA tiles per wavefront along M
  static constexpr int TN = kWaveN / 32;  // ... and along N
  static constexpr int kARows = kThreads / 8;   // A rows loaded per pass
  static constexpr int kAPasses = BM / kARows;  // 16-byte A chunks per thread per step
  static constexpr int kAPrefetch = PD_;        // steps of A in flight in registers
  static constexpr bool kPingPong = PP_;        // two-phase schedule (see the kernel)
  static constexpr int kBlocks = 2 * BN;        // weight blocks per 64-column step
  // Each thread decodes kBlocksPerThread whole blocks, or a half or a quarter of a
  // block when there are two or four times as many threads as blocks (kDecThreads).
  static constexpr int kBlocksPerThread = kBlocks > kThreads ? kBlocks / kThreads : 1;
  static constexpr int kDecThreads = kBlocks < kThreads ? kThreads / kBlocks : 1;
  static constexpr int kChunksPerBlock = 4 / kDecThreads;  // 16-byte chunks per block share
  static constexpr int kChunks = kBlocksPerThread * kChunksPerBlock;
  static constexpr int kABytes = BM * BK * 2;
  static constexpr int kWBytes = BN * BK * 2;
  static constexpr int kLutOffset = 2 * (kABytes + kWBytes);
  static constexpr int kLdsBytes = kLutOffset + (RFP4_GEMM_LUT ? 128 * 16 : 0);
  static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wavefront tile is whole MFMA tiles");
  static_assert(kARows % 16 == 0 && BM % kARows == 0 && kAPasses <= 8, "A loader shape");
  static_assert(kBlocks % kThreads == 0 || kThreads % kBlocks == 0, "decode split");
  static_assert(kDecThreads <= 4 && kBlocksPerThread <= 2, "decode split");
  static_assert(kAPrefetch == 1 || kAPrefetch == 2, "A prefetch depth");
  static_assert(kDecThreads == 1 || kBlocks % 64 == 0, "decode group uniform per wavefront");
  static_assert(kWaveM % 16 == 0 && kWaveN % 16 == 0, "fragment rows share a swizzle term");
  // Fragment reads use one base register per k slice and operand, plus an immediate
  // (buffer offset + tile row offset) when that fits the 16-bit field, else one base
  // register per buffer as well.
  static constexpr bool kSplitA = kABytes + (TM - 1) * 32 * 128 >= 65536;
  static constexpr bool kSplitW = kWBytes + (TN - 1) * 32 * 128 >= 65536;
};

// Main tiles: 0 = 256 x 256 with eight wavefronts (two per SIMD, 64 x 128 each);
// 1 = 512 x 128 with eight wavefronts (128 x 64 each; half the decode per flop);
// 2 = 256 x 256 with four wavefronts (one per SIMD, 128 x 128 each).
#ifndef RFP4_GEMM_MAIN
#define RFP4_GEMM_MAIN 0
#endif
#ifndef RFP4_GEMM_MAIN_PD
#define RFP4_GEMM_MAIN_PD 1
#endif
#ifndef RFP4_GEMM_PINGPONG
#define RFP4_GEMM_PINGPONG 1
#endif
using MainCfg = std::conditional_t<
    RFP4_GEMM_MAIN == 1, TileCfg<512, 128, 4, 2, RFP4_GEMM_MAIN_PD>,
    std::conditional_t<RFP4_GEMM_MAIN == 2, TileCfg<256, 256, 2, 2, RFP4_GEMM_MAIN_PD>,
                       std::conditional_t<RFP4_GEMM_PINGPONG != 0, TileCfg<256, 256, 4, 2, 2, true>,
                                          TileCfg<256, 256, 4, 2, RFP4_GEMM_MAIN_PD>>>>;
// Tail tiles: 5 = 128 x 128, four wavefronts (64 x 64 each, one per SIMD): measured
// against 4 (the ping-pong schedule, whose 32 x 64 wavefront tiles issue only 8 MFMAs
// per phase; counters: MFMA busy 22 % of the time) 18-22 % faster on all-tail plans;
// 4 = 128 x 128, eight wavefronts (32 x 64 each) on the ping-pong schedule;
// 0 = 128 x 64, four wavefronts (64 x 32 each); 1 = 128 x 64, eight
// wavefronts (32 x 32 each); 2 = 64 x 64, four wavefronts (32 x 32 each); 3 = 128 x 32,
// four wavefronts (32 x 32 each); 5 = 128 x 128, four wavefronts (64 x 64 each).
// RFP4_GEMM_TAIL_PD: steps of A prefetched.
#ifndef RFP4_GEMM_TAIL
#define RFP4_GEMM_TAIL 5
#endif
#ifndef RFP4_GEMM_TAIL_PD
#define RFP4_GEMM_TAIL_PD 1
#endif
using TailCfg = std::conditional_t<
    RFP4_GEMM_TAIL == 4, TileCfg<128, 128, 4, 2, 2, true>,
    std::conditional_t<RFP4_GEMM_TAIL == 5, TileCfg<128, 128, 2, 2, RFP4_GEMM_TAIL_PD>,
    std::conditional_t<
    RFP4_GEMM_TAIL == 1, TileCfg<128, 64, 4, 2, RFP4_GEMM_TAIL_PD>,
    std::conditional_t<
        RFP4_GEMM_TAIL == 2, TileCfg<64, 64, 2, 2, RFP4_GEMM_TAIL_PD>,
        std::conditional_t<RFP4_GEMM_TAIL == 3, TileCfg<128, 32, 4, 1, RFP4_GEMM_TAIL_PD>,
                           TileCfg<128, 64, 2, 2, RFP4_GEMM_TAIL_PD>>>>>>;

// LDS tiles are rows of 64 bf16 (128 bytes, eight 16-byte chunks); chunk c of row r
// is stored at chunk position c ^ ((r >> 1) & 7). A 16-byte access by 16 lanes covers
// 256 bytes of banks; with this swizzle the fragment reads (16 consecutive rows, one
// chunk), the A stores (two rows, eight chunks) and the weight stores (eight rows,
// chunks {c, c + 4}) all fall on distinct banks.
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  // Both values are exactly representable in bf16, so the conversion is exact.
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Packed bytes of one weight block held in registers between load and decode.
struct BlockRaw {
  uint4 qs;
  uint32_t sc;
};

template <int LAYOUT>
__device__ __forceinline__ BlockRaw load_block(const uint8_t* p) {
  BlockRaw b;
  b.qs = load16(p);
  if constexpr (LAYOUT == kDual) {
    uint16_t t;
    __builtin_memcpy(&t, p + 16, 2);
    b.sc = t;
  } else {
    b.sc = p[16];
  }
  return b;
}

#ifndef RFP4_GEMM_HW_SCALE
#define RFP4_GEMM_HW_SCALE 1
#endif

// Chunk C (weights 8C .. 8C+7) of one block as eight bf16 values c * S (exact).
// Chunks 0, 1 are the low nibbles of qs words 2C, 2C+1 (first half, scale e0);
// chunks 2, 3 the high nibbles of qs words 2(C-2), 2(C-2)+1 (second half, scale e1;
// the fast layout has one scale).
//
// The scale is taken either from the integer bit formula (any byte) or, for validated
// weights, from the hardware E4M3 converter applied to the byte's low seven bits, with
// codes of half-weights (the converter gives twice the decoded scale).
//
// Table decode: for each of the 128 values of a scale byte's low seven bits the table
// holds the bf16 encodings of the eight magnitudes times the decoded scale (exact), as
// a plane of low bytes (entries 0-3, 4-7) and a plane of high bytes. Four weights then
// take two v_perm_b32 that gather their low and high bytes by magnitude index, an OR
// of the sign bits into the high bytes (index 8 gives -0.0, harmless in the products)
// and two v_perm_b32 that interleave the planes into bf16 pairs.
template <int LAYOUT, int C>
__device__ __forceinline__ uint4 decode_chunk_table(const BlockRaw& b, const uint4& t) {
  const uint32_t q[4] = {b.qs.x, b.qs.y, b.qs.z, b.qs.w};
  uint32_t o[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t word = q[2 * (C & 1) + h];
    const uint32_t sel = (C < 2) ? (word & 0x07070707u) : ((word >> 4) & 0x07070707u);
    const uint32_t sign = (C < 2) ? ((word << 4) & 0x80808080u) : (word & 0x80808080u);
    const uint32_t lo = __builtin_amdgcn_perm(t.y, t.x, sel);
    const uint32_t hi = __builtin_amdgcn_perm(t.w, t.z, sel) | sign;
    o[2 * h] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    o[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

template <int LAYOUT, int C>
__device__ __forceinline__ uint4 decode_chunk(const BlockRaw& b, const uint4* tabs) {
#if RFP4_GEMM_LUT
  return decode_chunk_table<LAYOUT, C>(b, tabs[(C < 2 || LAYOUT == kFast) ? 0 : 1]);
#endif
  constexpr bool kFirst = C < 2 || LAYOUT == kFast;
#if RFP4_GEMM_HW_SCALE
  const uint32_t sc7 = b.sc & 0x7F7Fu;
  const float s = kFirst ? e4m3_hw<0>(sc7) : e4m3_hw<1>(sc7);
#else
  const float s = scale_exact(kFirst ? (b.sc & 0xFFu) : (b.sc >> 8));
#endif
  const uint32_t q[4] = {b.qs.x, b.qs.y, b.qs.z, b.qs.w};
  uint32_t o[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t word = q[2 * (C & 1) + h];
#if RFP4_GEMM_HW_SCALE
    const uint32_t codes = (C < 2) ? half_codes_low(word) : half_codes_high(word);
#else
    const uint32_t codes = (C < 2) ? codes_low(word) : codes_high(word);
#endif
    const f32x2 lo = pair_f32(codes, false);
    const f32x2 hi = pair_f32(codes, true);
    o[2 * h] = pack_bf16(lo.x * s, lo.y * s);
    o[2 * h + 1] = pack_bf16(hi.x * s, hi.y * s);
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

// Chunk CL of this thread's share of a block, stored at dst. With one thread per
// block the share is chunks 0..3; with two, group g owns chunks 2g, 2g + 1; with four,
// group g owns chunk g (the group is uniform over a wavefront).
template <int LAYOUT, typename Cfg, int CL>
__device__ __forceinline__ void decode_part(const BlockRaw& b, const uint4* tabs, char* dst,
                                            int grp) {
  uint4* d = reinterpret_cast<uint4*>(dst);
  if constexpr (Cfg::kDecThreads == 1) {
    *d = decode_chunk<LAYOUT, CL>(b, tabs);
  } else if constexpr (Cfg::kDecThreads == 2) {
    if (grp == 0)
      *d = decode_chunk<LAYOUT, CL>(b, tabs);
    else
      *d = decode_chunk<LAYOUT, CL + 2>(b, tabs);
  } else {
    if (grp == 0)
      *d = decode_chunk<LAYOUT, 0>(b, tabs);
    else if (grp == 1)
      *d = decode_chunk<LAYOUT, 1>(b, tabs);
    else if (grp == 2)
      *d = decode_chunk<LAYOUT, 2>(b, tabs);
    else
      *d = decode_chunk<LAYOUT, 3>(b, tabs);
  }
}

// XCD-aware tile order. Workgroups go to the 8 XCDs round-robin (workgroup b to XCD
// b mod 8) and each XCD has an L2 of its own. In the plain order (M tile = t mod
// m_tiles, N tile = t / m_tiles) with 8 M tiles, XCD x holds the slab of A of M tile x
// and streams every strip of W, so W crosses the fabric eight times. With mg > 0 (the
// launcher sets it when the tile counts divide), the XCDs form an mg x (8 / mg) grid:
// XCD x takes the M tiles of group x / (8 / mg) and the N strips of group x mod (8 / mg),
// in an order that keeps each resident round's tiles on a few slabs and strips, so A
// crosses the fabric 8 / mg times and W mg times. Every tile is computed the same way
// whichever workgroup runs it.
__device__ __forceinline__ void tile_coords(int t, int m_tiles, int tiles, int mg, int& mt, int64_t& nt) {
  if (mg > 0) {
    const int ng = 8 / mg;
    const int x = t & 7;
    const int j = t >> 3;
    const int mper = m_tiles / mg;
    mt = (x / ng) * mper + j % mper;
    nt = static_cast<int64_t>(x % ng) * ((tiles / m_tiles) / ng) + j / mper;
  } else {
    mt = t % m_tiles;
    nt = t / m_tiles;
  }
}

// Workgroup b computes tile t = b mod tiles, i.e. (t mod m_tiles, t / m_tiles), of the
// region of C whose columns start at n_base, over the part b / tiles of `splits`
// equal, even-length ranges of the k steps (k / 64 of them, rounded up to an even
// number, at least 2 * splits; KT marks k % 128 != 0). With one split the tile is rounded to bf16 and stored; with more, the
// fp32 accumulators go to partial[b] (BM x BN floats in accumulator order) for
// gemm_reduce_kernel. Rows and columns outside [0, m) x [0, n) are computed on clamped
// inputs and never stored.
template <int LAYOUT, typename Cfg, bool KT>
__global__ __launch_bounds__(Cfg::kThreads) void gemm_kernel(const uint8_t* __restrict__ w,
                                                             int n, int nb,
                                                             const uint16_t* __restrict__ a,
                                                             int m, int64_t lda,
                                                             uint16_t* __restrict__ c,
                                                             int64_t ldc, int m_tiles, int tiles,
                                                             int64_t n_base, int splits,
                                                             float* __restrict__ partial, int xcd_mg) {
  constexpr int BB = block_bytes(LAYOUT);
  constexpr int TM = Cfg::TM;
  constexpr int TN = Cfg::TN;
  // LDS: A buffers 0 and 1, then W buffers 0 and 1, so that every fragment read is one
  // of a few per-lane base registers plus an immediate offset below 64 KB.
  constexpr int kW0 = 2 * Cfg::kABytes;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / Cfg::WN;
  const int wn = wid % Cfg::WN;
  const int tile_id = static_cast<int>(blockIdx.x) % tiles;
  const int split = static_cast<int>(blockIdx.x) / tiles;
  int mt;
  int64_t nt;
  tile_coords(tile_id, m_tiles, tiles, xcd_mg, mt, nt);
  const int m0 = mt * Cfg::BM;
  const int64_t n0 = n_base + nt * Cfg::BN;
  const int64_t rowbytes = static_cast<int64_t>(nb) * BB;
  // BK = 64 = two blocks; steps come in pairs. With KT (k tail: nb not a multiple of
  // four) the last pair reaches past k, and its A chunks and weight blocks beyond k
  // are read as zeros.
  const int half_steps = KT ? (nb + 3) / 4 : nb / 4;
  const int s_begin = 2 * static_cast<int>(static_cast<int64_t>(split) * half_steps / splits);
  const int s_end = 2 * static_cast<int>(static_cast<int64_t>(split + 1) * half_steps / splits);
  const int s_last = s_end - 1;

  // A loader: thread -> 16-byte chunk (t % 8) of rows t/8 + kARows * i (eight threads
  // cover a row's 128 contiguous bytes); staged in registers, written to the swizzled
  // LDS tile after the MFMAs of the current step. kARows is a multiple of 16, so the
  // rows of a thread share one swizzle term.
  constexpr int AP = Cfg::kAPasses;
  const int a_row0 = tid >> 3;
  const int a_chunk = tid & 7;
  struct AChunks {
    uint4 v[AP];
  };
  const uint16_t* a_p[AP];
#pragma unroll
  for (int i = 0; i < AP; ++i)  // rows past m are clamped to row m - 1, never stored
    a_p[i] = a + a_chunk * 8 + min(m0 + a_row0 + Cfg::kARows * i, m - 1) * lda;
  auto load_a = [&](int s) {
    AChunks r;
    if constexpr (KT) {
      // Past k: load column 0 of the row instead (always in bounds) and zero the chunk.
      const bool ok = s * BK + a_chunk * 8 < nb * 32;
      const int off = ok ? s * BK : -a_chunk * 8;
#pragma unroll
      for (int i = 0; i < AP; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(a_p[i] + off);
        r.v[i] = ok ? v : uint4{0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int i = 0; i < AP; ++i) r.v[i] = *reinterpret_cast<const uint4*>(a_p[i] + s * BK);
    }
    return r;
  };
  char* const a_st = smem + a_row0 * 128 + (swz_chunk(a_row0, a_chunk) << 4);
  auto store_a = [&](const AChunks& r, int buf) {
#pragma unroll
    for (int i = 0; i < AP; ++i)
      *reinterpret_cast<uint4*>(a_st + buf * Cfg::kABytes + i * Cfg::kARows * 128) = r.v[i];
  };

  // W loader: thread -> blocks w_idx + kThreads q (q < kBlocksPerThread) of the step;
  // block index bi covers weight row bi / 2, block bi % 2 of the step (columns
  // 32 (bi % 2) .. 32 (bi % 2) + 31 of the 64).
  constexpr int BP = Cfg::kBlocksPerThread;
  constexpr int CPB = Cfg::kChunksPerBlock;
  const int w_idx = tid % Cfg::kBlocks;
  const int w_grp = __builtin_amdgcn_readfirstlane(tid / Cfg::kBlocks);
  const uint8_t* w_row[BP];
  char* w_st[BP][CPB];
#pragma unroll
  for (int q = 0; q < BP; ++q) {
    const int bi = w_idx + Cfg::kThreads * q;
    const int r = bi >> 1;
    const int blk = bi & 1;
    w_row[q] = w + min(n0 + r, static_cast<int64_t>(n) - 1) * rowbytes + blk * BB;
#pragma unroll
    for (int j = 0; j < CPB; ++j) {
      const int cc = 4 * blk + w_grp * CPB + j;  // chunk of the 64-column LDS row
      w_st[q][j] = smem + kW0 + r * 128 + (swz_chunk(r, cc) << 4);
    }
  }
  struct WRaw {
    BlockRaw b[BP];
  };
  auto load_w = [&](int s) {
    WRaw r;
#pragma unroll
    for (int q = 0; q < BP; ++q) {
      if constexpr (KT) {
        // Past k: load the row's first block instead and zero it (index 0, scale 0).
        const int blk = (w_idx + Cfg::kThreads * q) & 1;
        const bool ok = 2 * s + blk < nb;
        const BlockRaw b = load_block<LAYOUT>(w_row[q] + (ok ? s * 2 * BB : -blk * BB));
        r.b[q].qs = ok ? b.qs : uint4{0u, 0u, 0u, 0u};
        r.b[q].sc = ok ? b.sc : 0u;
      } else {
        r.b[q] = load_block<LAYOUT>(w_row[q] + s * 2 * BB);
      }
    }
    return r;
  };
  // Decode tables of the scale bytes of this thread's blocks (entries e0, e1).
  struct WTab {
    uint4 t[BP][2];
  };
  auto load_tabs = [&](const WRaw& wr) {
    WTab r;
#pragma unroll
    for (int q = 0; q < BP; ++q) {
#if RFP4_GEMM_LUT
      const uint32_t sc = wr.b[q].sc;
      const char* lut = smem + Cfg::kLutOffset;
      r.t[q][0] = *reinterpret_cast<const uint4*>(lut + ((sc & 0x7Fu) << 4));
      r.t[q][1] = LAYOUT == kDual ? *reinterpret_cast<const uint4*>(lut + (((sc >> 8) & 0x7Fu) << 4))
                                  : r.t[q][0];
#else
      r.t[q][0] = r.t[q][1] = uint4{0u, 0u, 0u, 0u};
#endif
    }
    return r;
  };
  // Local chunk J = q * CPB + j of this thread's decode work for one step.
  auto decode_to = [&](const WRaw& wr, const WTab& tb, int buf, auto j_c) {
    constexpr int J = decltype(j_c)::value;
    constexpr int q = J / CPB;
    constexpr int j = J % CPB;
    decode_part<LAYOUT, Cfg, j>(wr.b[q], tb.t[q], w_st[q][j] + buf * Cfg::kWBytes, w_grp);
  };
  // The local chunks decoded alongside k slice kk: [kk C / 4, (kk + 1) C / 4) with C =
  // kChunks, so the decode work is spread evenly over the four slices of a step.
  auto decode_slot = [&](const WRaw& wr, const WTab& tb, int buf, auto kk_c) {
    constexpr int kk = decltype(kk_c)::value;
    constexpr int J0 = kk * Cfg::kChunks / 4;
    constexpr int J1 = (kk + 1) * Cfg::kChunks / 4;
    static_assert(J1 - J0 <= 2, "at most two chunks per k slice");
    if constexpr (J0 < J1) decode_to(wr, tb, buf, std::integral_constant<int, J0>{});
    if constexpr (J0 + 1 < J1) decode_to(wr, tb, buf, std::integral_constant<int, J0 + 1>{});
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // A in flight: with prefetch depth PD > 1, the A chunks of step s + PD are loaded
  // into ring slot s % PD at the start of step s, and slot (s + 1) % PD (stage s + 1)
  // is written to LDS at its end.
  constexpr int PD = Cfg::kAPrefetch;
  AChunks a_ring[PD];

  // Prologue: stage 0 in LDS, the weights of stage 1 and the A chunks of stages
  // 1 .. PD - 1 in registers.
  {
    const AChunks a0 = load_a(s_begin);
    const WRaw b0 = load_w(s_begin);
#if RFP4_GEMM_LUT
    // Decode table: entry e (the low seven bits of a scale byte) holds bf16(m * S(e))
    // for the magnitudes m = 0, 1, 2, 3, 4, 6, 8, 10 as a low-byte and a high-byte
    // plane. Every product is exactly representable, so truncating fp32 is exact.
    if (tid < 128) {
      const float sv = scale_exact(static_cast<uint32_t>(tid));
      const float mags[8] = {0.f, 1.f, 2.f, 3.f, 4.f, 6.f, 8.f, 10.f};
      uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t bits = __float_as_uint(mags[i] * sv) >> 16;
        lo[i >> 2] |= (bits & 0xFFu) << (8 * (i & 3));
        hi[i >> 2] |= (bits >> 8) << (8 * (i & 3));
      }
      *reinterpret_cast<uint4*>(smem + Cfg::kLutOffset + 16 * tid) = uint4{lo[0], lo[1], hi[0], hi[1]};
    }
    __syncthreads();
#endif
    const WTab t0 = load_tabs(b0);
    store_a(a0, 0);
    decode_slot(b0, t0, 0, std::integral_constant<int, 0>{});
    decode_slot(b0, t0, 0, std::integral_constant<int, 1>{});
    decode_slot(b0, t0, 0, std::integral_constant<int, 2>{});
    decode_slot(b0, t0, 0, std::integral_constant<int, 3>{});
  }
  WRaw w_next = load_w(min(s_begin + 1, s_last));
#pragma unroll
  for (int p = 1; p < PD; ++p) a_ring[p] = load_a(min(s_begin + p, s_last));
  __syncthreads();

  // Fragment addresses. Lane (fr, fk) reads row fr of each 32-row MFMA tile and the
  // 8-column half fk of a 16-column k slice kk, i.e. logical chunk 2 kk + fk. The rows
  // of a lane's fragments differ by multiples of 16 and share the swizzle term.
  const int fr = lane & 31;
  const int fk = lane >> 5;
  constexpr int NBA = Cfg::kSplitA ? 2 : 1;
  constexpr int NBW = Cfg::kSplitW ? 2 : 1;
  const char* a_frag[NBA][4];
  const char* w_frag[NBW][4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int pc = swz_chunk(fr, 2 * kk + fk) << 4;
#pragma unroll
    for (int bu = 0; bu < NBA; ++bu)
      a_frag[bu][kk] = smem + bu * Cfg::kABytes + (wm * Cfg::kWaveM + fr) * 128 + pc;
#pragma unroll
    for (int bu = 0; bu < NBW; ++bu)
      w_frag[bu][kk] = smem + kW0 + bu * Cfg::kWBytes + (wn * Cfg::kWaveN + fr) * 128 + pc;
  }

  // One step: multiply stage `cur` out of LDS while the next stage is prepared in the
  // other buffer. The loop below runs two steps per iteration so that the buffer index
  // is a compile-time constant and every LDS address is a base register plus an
  // immediate. On the last steps the prefetches are clamped to the last stage and only
  // refill the buffer that is no longer read.
  auto step = [&](auto u_c, int s) {
    constexpr int U = decltype(u_c)::value;  // s mod the unroll factor
    constexpr int cur = U & 1;
    // Issue order matters: the A loads first and the weight loads after them, so that
    // storing A at the end of the step waits only for the A loads (vmcnt counts in
    // issue order); the scheduling barrier keeps the compiler from sinking the loads.
    a_ring[U % PD] = load_a(min(s + PD, s_last));
    const WRaw w_after = load_w(min(s + 2, s_last));  // two steps ahead
    __builtin_amdgcn_sched_barrier(0);
    const WTab tn = load_tabs(w_next);
    bf16x8 af[2][TM], bfr[2][TN];
    auto load_frags = [&](int kk, int slot) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[slot][i] = *reinterpret_cast<const bf16x8*>(
            Cfg::kSplitA ? a_frag[NBA - 1 < cur ? 0 : cur][kk] + i * 32 * 128
                         : a_frag[0][kk] + cur * Cfg::kABytes + i * 32 * 128);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[slot][j] = *reinterpret_cast<const bf16x8*>(
            Cfg::kSplitW ? w_frag[NBW - 1 < cur ? 0 : cur][kk] + j * 32 * 128
                         : w_frag[0][kk] + cur * Cfg::kWBytes + j * 32 * 128);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bfr[slot][j], acc[i][j], 0, 0, 0);
    };
    // k slice kk: fragments of kk+1 are read while the MFMAs of kk run, and a share of
    // the next stage's weights is decoded alongside.
    // Scheduling fences keep this order: the fragments of slice kk + 1 are read before
    // the MFMAs of slice kk are issued, so each read has a whole slice of MFMAs to land
    // (left alone, the compiler moves the reads next to their uses and exposes the LDS
    // latency once per slice).
#ifndef RFP4_GEMM_FENCE
#define RFP4_GEMM_FENCE 1
#endif
    auto fence = [&]() {
      if constexpr (RFP4_GEMM_FENCE != 0 || TM * TN >= 16) __builtin_amdgcn_sched_barrier(0);
    };
    load_frags(0, 0);
    load_frags(1, 1);
    fence();
    mfmas(0);
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 0>{});
    fence();
    load_frags(2, 0);
    fence();
    mfmas(1);
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 1>{});
    fence();
    load_frags(3, 1);
    fence();
    mfmas(0);
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 2>{});
    fence();
    mfmas(1);
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 3>{});
    __builtin_amdgcn_sched_barrier(0);
    store_a(a_ring[(U + 1) % PD], cur ^ 1);
    w_next = w_after;
    __syncthreads();
  };
  // Ping-pong schedule (eight wavefronts, two per SIMD). Waves 0-3 and 4-7 sit on the
  // same four SIMDs; each step has two phases separated by barriers. In one phase a
  // group issues its 32 MFMAs on stage s (fragments read one slice ahead) while the
  // other group prepares its half of stage s + 1 (A chunks and decoded weights into the
  // other buffer, loads for later stages); in the next phase the roles swap. The MFMA
  // pipe of every SIMD is fed by one wave while the other issues VALU and memory work.
  // The weight rows and A rows a thread prepares lie in its group's half of the tile
  // (thread t handles weight row t / 2 and A rows t / 8 + kARows i).
#ifndef RFP4_GEMM_SETPRIO
#define RFP4_GEMM_SETPRIO 1
#endif
  auto mfma_block = [&](auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    // The wave issuing MFMAs takes issue priority over its SIMD partner's VALU work.
    if constexpr (RFP4_GEMM_SETPRIO) __builtin_amdgcn_s_setprio(1);
    bf16x8 af[2][TM], bfr[2][TN];
    auto load_frags = [&](int kk, int slot) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[slot][i] = *reinterpret_cast<const bf16x8*>(
            Cfg::kSplitA ? a_frag[NBA - 1 < cur ? 0 : cur][kk] + i * 32 * 128
                         : a_frag[0][kk] + cur * Cfg::kABytes + i * 32 * 128);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[slot][j] = *reinterpret_cast<const bf16x8*>(
            Cfg::kSplitW ? w_frag[NBW - 1 < cur ? 0 : cur][kk] + j * 32 * 128
                         : w_frag[0][kk] + cur * Cfg::kWBytes + j * 32 * 128);
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bfr[slot][j], acc[i][j], 0, 0, 0);
    };
    load_frags(0, 0);
    load_frags(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(2, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(3, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RFP4_GEMM_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };
  // Prepare stage s + 1 in buffer (s + 1) % 2: loads for A(s + PD) and W(s + 2) are
  // issued first, then A(s + 1) (loaded PD - 1 steps earlier) is stored and W(s + 1)
  // (loaded one step earlier) decoded.
  auto prep_block = [&](auto u_c, int s) {
    constexpr int U = decltype(u_c)::value;
    constexpr int cur = U & 1;
    a_ring[U % PD] = load_a(min(s + PD, s_last));
    const WRaw w_after = load_w(min(s + 2, s_last));
    __builtin_amdgcn_sched_barrier(0);
    const WTab tn = load_tabs(w_next);
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 0>{});
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 1>{});
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 2>{});
    decode_slot(w_next, tn, cur ^ 1, std::integral_constant<int, 3>{});
    store_a(a_ring[(U + 1) % PD], cur ^ 1);
    w_next = w_after;
    __builtin_amdgcn_sched_barrier(0);
  };
  // Each group runs its own straight-line loop; both loops execute the same sequence
  // of workgroup barriers (two per step), which pairs them phase by phase.
  auto pp_step = [&](auto u_c, int s, auto second_c) {
    constexpr int U = decltype(u_c)::value;
    constexpr auto cur_c = std::integral_constant<int, (U & 1)>{};
#ifndef RFP4_GEMM_MID_BARRIER
#define RFP4_GEMM_MID_BARRIER 1
#endif
    if constexpr (!decltype(second_c)::value) {
      mfma_block(cur_c);
      if constexpr (RFP4_GEMM_MID_BARRIER) __syncthreads();
      prep_block(u_c, s);
      __syncthreads();
    } else {
      prep_block(u_c, s);
      if constexpr (RFP4_GEMM_MID_BARRIER) __syncthreads();
      mfma_block(cur_c);
      __syncthreads();
    }
  };

  // The range [s_begin, s_end) has even bounds, so stage s lives in buffer s % 2 and
  // ring slot s % PD.
  if constexpr (Cfg::kPingPong) {
    static_assert(PD == 2, "the ping-pong schedule keeps two stages of A in registers");
    if (wid < Cfg::WM * Cfg::WN / 2) {  // uniform over a wavefront
      for (int s = s_begin; s < s_end; s += 2) {
        pp_step(std::integral_constant<int, 0>{}, s, std::false_type{});
        pp_step(std::integral_constant<int, 1>{}, s + 1, std::false_type{});
      }
    } else {
      for (int s = s_begin; s < s_end; s += 2) {
        pp_step(std::integral_constant<int, 0>{}, s, std::true_type{});
        pp_step(std::integral_constant<int, 1>{}, s + 1, std::true_type{});
      }
    }
  } else {
    for (int s = s_begin; s < s_end; s += 2) {
      step(std::integral_constant<int, 0>{}, s);
      step(std::integral_constant<int, 1>{}, s + 1);
    }
  }

  // Epilogue. 32x32 accumulator layout: register e of lane l holds row
  // 8*(e/4) + 4*(l/32) + (e%4), column l%32 of the MFMA tile.
  if (partial != nullptr) {
    // Partial sums, stored as float4 groups (registers 4 e4 .. 4 e4 + 3) at index
    // ((wave * TM + i) * TN + j) * 4 + e4 of 64 lanes each: 1 KB contiguous per store.
    float4* dst = reinterpret_cast<float4*>(partial + static_cast<int64_t>(blockIdx.x) * Cfg::BM * Cfg::BN);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          dst[(((wid * TM + i) * TN + j) * 4 + e4) * 64 + lane] =
              make_float4(acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                          acc[i][j][4 * e4 + 3]);
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t gn = n0 + wn * Cfg::kWaveN + j * 32 + (lane & 31);
      if (gn >= n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gm = m0 + wm * Cfg::kWaveM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (gm < m) c[gm * ldc + gn] = bf16_rne(acc[i][j][e]);
      }
    }
  }
}

// Sums the `splits` partial tiles of each of `tiles` tiles (split order 0, 1, ...),
// rounds to bf16 and stores the tile's part of C. Thread g handles float4 group g of
// the accumulator order written by gemm_kernel.
template <typename Cfg>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ partial,
                                                          int splits, int tiles, int m_tiles,
                                                          int64_t n_base, int m, int n,
                                                          uint16_t* __restrict__ c, int64_t ldc,
                                                          int xcd_mg) {
  constexpr int kGroups = Cfg::BM * Cfg::BN / 4;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= static_cast<int64_t>(tiles) * kGroups) return;
  const int tile = static_cast<int>(g / kGroups);
  const int idx = static_cast<int>(g % kGroups);
  const float4* p = reinterpret_cast<const float4*>(partial);
  float4 sum = p[static_cast<int64_t>(tile) * kGroups + idx];
  for (int sp = 1; sp < splits; ++sp) {
    const float4 v = p[(static_cast<int64_t>(sp) * tiles + tile) * kGroups + idx];
    sum.x += v.x;
    sum.y += v.y;
    sum.z += v.z;
    sum.w += v.w;
  }
  const int lane = idx % 64;
  int r = idx / 64;
  const int e4 = r % 4;
  r /= 4;
  const int j = r % Cfg::TN;
  r /= Cfg::TN;
  const int i = r % Cfg::TM;
  const int wid = r / Cfg::TM;
  const int wm = wid / Cfg::WN;
  const int wn = wid % Cfg::WN;
  int mt;
  int64_t nt;
  tile_coords(tile, m_tiles, tiles, xcd_mg, mt, nt);
  const int m0 = mt * Cfg::BM;
  const int64_t n0 = n_base + nt * Cfg::BN;
  const int64_t gn = n0 + wn * Cfg::kWaveN + j * 32 + (lane & 31);
  if (gn >= n) return;
  const int row0 = m0 + wm * Cfg::kWaveM + i * 32 + 8 * e4 + 4 * (lane >> 5);
  const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (row0 + q < m) c[(row0 + q) * ldc + gn] = bf16_rne(v[q]);
}

template <typename Cfg, bool KT>
const void* kernel_ptr(int layout) {
  return layout == kDual ? reinterpret_cast<const void*>(&gemm_kernel<kDual, Cfg, KT>)
                         : reinterpret_cast<const void*>(&gemm_kernel<kFast, Cfg, KT>);
}

// Raises the dynamic-LDS limit of both configurations once per device; threads that
// race repeat the same idempotent calls.
hipError_t ensure_attributes(int layout) {
  static std::atomic<bool> done[64][2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < 64;
  if (cached && done[dev][layout].load(std::memory_order_acquire)) return hipSuccess;
  const void* fns[4] = {kernel_ptr<MainCfg, false>(layout), kernel_ptr<MainCfg, true>(layout),
                        kernel_ptr<TailCfg, false>(layout), kernel_ptr<TailCfg, true>(layout)};
  const int lds[4] = {MainCfg::kLdsBytes, MainCfg::kLdsBytes, TailCfg::kLdsBytes, TailCfg::kLdsBytes};
  for (int i = 0; i < 4; ++i) {
    e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, lds[i]);
    if (e != hipSuccess) return e;
  }
  if (cached) done[dev][layout].store(true, std::memory_order_release);
  return hipSuccess;
}

// Columns [n_base, n_end) of C for rows [0, m), tiled with configuration Cfg, each tile's
// k range split `splits` ways (partial sums in `partial`, then reduced) when splits > 1.
template <typename Cfg>
hipError_t launch_region(const uint8_t* w, int layout, int n, int nb, const uint16_t* a, int m,
                         int64_t lda, uint16_t* c, int64_t ldc, int64_t n_base, int64_t n_end,
                         int splits, float* partial, hipStream_t stream) {
  if (n_end <= n_base) return hipSuccess;
  const int m_tiles = (m + Cfg::BM - 1) / Cfg::BM;
  // At most 2^39 elements of C (checked by the API): at most 2^26 tiles.
  const int64_t n_tiles = (n_end - n_base + Cfg::BN - 1) / Cfg::BN;
  const int tiles = static_cast<int>(m_tiles * n_tiles);
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(tiles) * splits));
  float* part = splits > 1 ? partial : nullptr;
  // XCD grouping (tile_coords): the mg x (8 / mg) grid that moves the fewest bytes of A
  // and W across the fabric, A crossing 8 / mg times and W mg times; 0 (plain order) when
  // the tile counts do not divide.
  int mg = 0;
#ifndef RFP4_GEMM_XCD
#define RFP4_GEMM_XCD 1
#endif
  // The grid assumes 8 XCDs of 32 CUs (gfx950 as one partition, 256 CUs); a device
  // exposing another CU count (a partitioned GPU) keeps the plain order, which is equally
  // correct, only without the locality.
  if (RFP4_GEMM_XCD && tiles % 8 == 0 && device_cu_count() == 256) {
    const double a_bytes = static_cast<double>(m) * nb * 64;
    const double w_bytes = static_cast<double>(n_end - n_base) * nb * block_bytes(layout);
    double best = 0.0;
    for (int g = 1; g <= 8; g *= 2) {
      if (m_tiles % g != 0 || n_tiles % (8 / g) != 0) continue;
      const double cost = a_bytes * (8 / g) + w_bytes * g;
      if (mg == 0 || cost < best) {
        best = cost;
        mg = g;
      }
    }
  }
#define RFP4_GEMM_LAUNCH(L, KT)                                                     \
  gemm_kernel<L, Cfg, KT><<<grid, dim3(Cfg::kThreads), Cfg::kLdsBytes, stream>>>( \
      w, n, nb, a, m, lda, c, ldc, m_tiles, tiles, n_base, splits, part, mg)
  const bool kt = nb % 4 != 0;
  if (layout == kDual) {
    if (kt) RFP4_GEMM_LAUNCH(kDual, true); else RFP4_GEMM_LAUNCH(kDual, false);
  } else {
    if (kt) RFP4_GEMM_LAUNCH(kFast, true); else RFP4_GEMM_LAUNCH(kFast, false);
  }
#undef RFP4_GEMM_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t groups = static_cast<int64_t>(tiles) * (Cfg::BM * Cfg::BN / 4);
  gemm_reduce_kernel<Cfg><<<dim3(static_cast<unsigned>((groups + 255) / 256)), dim3(256), 0, stream>>>(
      partial, splits, tiles, m_tiles, n_base, m, n, c, ldc, mg);
  return hipGetLastError();
}

// Cost model of a plan, fitted to measured launches on MI355X (2048 x 17408 x 5120,
// 4096 x 17408 x 5120, 2048 x 5120 x 17408, 2048 x 5120 x 6144, 2048 x 6144 x 5120,
// 2048 x 1024 x 5120, 512 x 17408 x 5120 under every plan): a round of workgroups (one
// per CU) costs kMainUsPerK (256 x 256 tiles) or kTailUsPerK (128 x 128 tiles) times its
// k columns; a last, partial round filling a fraction f of the CUs costs f^kPartialExp
// of a full one (fewer busy CUs run faster); a split adds a reduction that moves its
// partial sums at kReduceBytesPerUs plus kReduceFixedUs. It ranks the measured plans of
// those shapes in the measured order of their best.
constexpr double kMainUsPerK = 0.030;
constexpr double kTailUsPerK = 0.0102;
constexpr double kPartialExp = 0.4;
constexpr double kReduceBytesPerUs = 3.8e6;
constexpr double kReduceFixedUs = 5.0;

struct Plan {
  int64_t tail_strips;  // trailing 256-column strips of C computed with tail tiles
  int splits;           // k-range split of each tail tile
  int64_t tail_tiles;   // tail tiles (before the split)
  int main_splits = 1;  // k-range split of each main tile
  int64_t main_tiles = 0;
};

inline double rounds(int64_t workgroups, int cus) {
  const int64_t full = workgroups / cus;
  const double frac = static_cast<double>(workgroups % cus) / cus;
  return static_cast<double>(full) + (frac > 0.0 ? std::pow(frac, kPartialExp) : 0.0);
}

// Chooses the tail strips and the splits of main and tail tiles with the lowest modelled
// time, among plans whose partial sums fit max_partial_bytes. A forced plan (rfp4_force)
// selects all-main tiles, all-tail tiles with a given split, or all-main tiles with a
// given split (so tests cover every path at small sizes), or restricts the choice to
// plans without a split.
Plan choose_plan(int64_t m, int64_t n, int nb, int cus, int forced, double max_partial_bytes) {
  const int64_t strips = (n + MainCfg::BN - 1) / MainCfg::BN;
  const int64_t mt = (m + MainCfg::BM - 1) / MainCfg::BM;
  const int64_t slabs = (m + TailCfg::BM - 1) / TailCfg::BM;
  auto tail_tiles = [&](int64_t t) {
    const int64_t cols = n - (strips - t) * MainCfg::BN;
    return t > 0 ? slabs * ((cols + TailCfg::BN - 1) / TailCfg::BN) : 0;
  };
  const int max_split = (nb + 3) / 4;  // each split needs at least two 64-column steps
  const double k = 32.0 * nb;
  if (forced == RFP4_GEMM_PLAN_MAIN) return Plan{0, 1, 0, 1, mt * strips};
  if (forced >= RFP4_GEMM_PLAN_MSPLIT2 && forced <= RFP4_GEMM_PLAN_MSPLIT4)
    return Plan{0, 1, 0, std::min(forced - RFP4_GEMM_PLAN_MSPLIT2 + 2, max_split), mt * strips};
  if (forced >= RFP4_GEMM_PLAN_TAIL && forced <= RFP4_GEMM_PLAN_TAIL4) {
    int sp = forced == RFP4_GEMM_PLAN_TAIL ? 1 : (forced == RFP4_GEMM_PLAN_TAIL2 ? 2 : 4);
    if (sp > max_split) sp = max_split;
    return Plan{strips, sp, tail_tiles(strips)};
  }
  const bool allow_split = forced != RFP4_GEMM_PLAN_NOSPLIT;
  auto reduce_us = [](int64_t tiles, int sp, int tile_elems) {
    return sp > 1 ? (static_cast<double>(tiles) * tile_elems * (4.0 * sp + 2.0)) / kReduceBytesPerUs +
                        kReduceFixedUs
                  : 0.0;
  };
  auto partial_ok = [&](int64_t tiles, int sp, int tile_elems) {
    return sp == 1 || static_cast<double>(tiles) * sp * tile_elems * 4.0 <= max_partial_bytes;
  };
  Plan best{0, 1, 0, 1, mt * strips};
  double best_cost = 1e300;
  const int64_t max_tail = strips < 256 ? strips : 256;
  for (int64_t t = 0; t <= max_tail; ++t) {
    const int64_t main_tiles = mt * (strips - t);
    const int64_t tt = tail_tiles(t);
    for (int spm = 1; spm <= 4; ++spm) {
      if (spm > 1 && (!allow_split || spm > max_split || main_tiles == 0)) break;
      if (!partial_ok(main_tiles, spm, MainCfg::BM * MainCfg::BN)) break;
      const double cm = main_tiles > 0 ? kMainUsPerK * k / spm * rounds(main_tiles * spm, cus) +
                                             reduce_us(main_tiles, spm, MainCfg::BM * MainCfg::BN)
                                       : 0.0;
      for (int sp = 1; sp <= 8; sp *= 2) {
        if (sp > 1 && (!allow_split || sp > max_split || tt == 0)) break;
        if (!partial_ok(tt, sp, TailCfg::BM * TailCfg::BN)) break;
        const double ct = tt > 0 ? kTailUsPerK * k / sp * rounds(tt * sp, cus) +
                                       reduce_us(tt, sp, TailCfg::BM * TailCfg::BN)
                                 : 0.0;
        const double pbytes = (spm > 1 ? static_cast<double>(main_tiles) * spm * MainCfg::BM * MainCfg::BN * 4.0 : 0.0) +
                              (sp > 1 ? static_cast<double>(tt) * sp * TailCfg::BM * TailCfg::BN * 4.0 : 0.0);
        if (pbytes > max_partial_bytes) continue;
        if (cm + ct < best_cost - 1e-9) {
          best_cost = cm + ct;
          best = Plan{t, sp, tt, spm, main_tiles};
        }
      }
    }
  }
  return best;
}

}  // namespace

namespace {

// The GEMM over all rows, in chunks of rows so each grid stays within 2^31 workgroups.
// `get_ws(bytes, &ptr)` provides the partial-sum buffer of a split plan (false: none,
// and the chunk then runs its plan unsplit); plans are chosen among those whose
// partial sums fit max_partial_bytes.
template <typename GetWs>
hipError_t run_gemm(const uint8_t* w, int layout, int64_t n, int64_t k, const uint16_t* a,
                    int64_t m, int64_t lda, uint16_t* c, int64_t ldc, int forced,
                    double max_partial_bytes, GetWs get_ws, hipStream_t stream) {
  // Any k % 32 == 0: the kernel runs two 64-column steps per iteration, and when
  // k % 128 != 0 its k-tail variant zero-fills the last pair past k.
  const int nb = static_cast<int>(k / 32);
  hipError_t e = ensure_attributes(layout);
  if (e != hipSuccess) return e;
  const int cus = device_cu_count();
  const int64_t strips = (n + MainCfg::BN - 1) / MainCfg::BN;
  const int64_t max_m = int64_t(1) << 20;
  for (int64_t m_off = 0; m_off < m; m_off += max_m) {
    const int mc = static_cast<int>(m - m_off < max_m ? m - m_off : max_m);
    Plan plan = choose_plan(mc, n, nb, cus, forced, max_partial_bytes);
    float* partial = nullptr;       // tail partial sums
    float* partial_main = nullptr;  // main partial sums (before the tail's)
    const size_t main_bytes = plan.main_splits > 1 ? static_cast<size_t>(plan.main_tiles) * plan.main_splits *
                                                         MainCfg::BM * MainCfg::BN * sizeof(float)
                                                   : 0;
    const size_t tail_bytes = plan.splits > 1 ? static_cast<size_t>(plan.tail_tiles) * plan.splits *
                                                    TailCfg::BM * TailCfg::BN * sizeof(float)
                                              : 0;
    if (main_bytes + tail_bytes > 0) {
      float* ws = nullptr;
      if (!get_ws(main_bytes + tail_bytes, &ws)) {
        plan.splits = 1;  // no workspace (graph capture or no memory): run every tile unsplit
        plan.main_splits = 1;
      } else {
        partial_main = ws;
        partial = ws + main_bytes / sizeof(float);
      }
    }
    const int64_t n_split = (strips - plan.tail_strips) * MainCfg::BN;
    const uint16_t* ap = a + m_off * lda;
    uint16_t* cp = c + m_off * ldc;
    e = launch_region<MainCfg>(w, layout, static_cast<int>(n), nb, ap, mc, lda, cp, ldc, 0, n_split,
                               plan.main_splits, partial_main, stream);
    if (e != hipSuccess) return e;
    e = launch_region<TailCfg>(w, layout, static_cast<int>(n), nb, ap, mc, lda, cp, ldc, n_split, n,
                               plan.splits, partial, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm(const uint8_t* w, int layout, int64_t n, int64_t k, const uint16_t* a,
                       int64_t m, int64_t lda, uint16_t* c, int64_t ldc, const Force& force,
                       hipStream_t stream) {
  auto get_ws = [&](size_t bytes, float** out) {
    return stream_workspace(kWorkspaceGemm, stream, bytes, false, reinterpret_cast<void**>(out)) == hipSuccess;
  };
  return run_gemm(w, layout, n, k, a, m, lda, c, ldc, force.gemm_plan, 512.0 * 1024 * 1024, get_ws, stream);
}

// ---------------------------------------------------------------- allocation-free GEMM
//
// The partial sums of split plans live in `scratch`, a static device array (one copy
// per GPU the library runs on, kept until the process ends) instead of a workspace, so
// rfp4_gemm_noalloc calls no allocator. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): its device address is
// looked up once per device with that device current and kept.
static __device__ __align__(256) float scratch[kGemmScratchBytes / sizeof(float)];

namespace {

// Device address of `scratch` on the current device (looked up on the first call per
// device, under a lock; threads that come later read the kept address).
hipError_t scratch_address(float** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

}  // namespace

// Partial-sum bytes of the plan rfp4_gemm_noalloc would run for this shape (0 = no
// split); the same planner as launch_gemm_noalloc, so a caller can reject a shape
// before any launch.
double gemm_noalloc_plan_bytes(int64_t n, int64_t k, int64_t m, const Force& force) {
  const int nb = static_cast<int>(k / 32);
  const int cus = device_cu_count();
  const int64_t max_m = int64_t(1) << 20;
  double need = 0.0;
  for (int64_t m_off = 0; m_off < m; m_off += max_m) {
    const int mc = static_cast<int>(m - m_off < max_m ? m - m_off : max_m);
    const Plan plan = choose_plan(mc, n, nb, cus, force.gemm_plan, static_cast<double>(kGemmScratchBytes));
    const double b = (plan.main_splits > 1 ? static_cast<double>(plan.main_tiles) * plan.main_splits *
                                                 MainCfg::BM * MainCfg::BN * 4.0
                                           : 0.0) +
                     (plan.splits > 1 ? static_cast<double>(plan.tail_tiles) * plan.splits *
                                            TailCfg::BM * TailCfg::BN * 4.0
                                      : 0.0);
    need = std::max(need, b);
  }
  return need;
}

hipError_t launch_gemm_noalloc(const uint8_t* w, int layout, int64_t n, int64_t k, const uint16_t* a,
                               int64_t m, int64_t lda, uint16_t* c, int64_t ldc, const Force& force,
                               hipStream_t stream) {
  float* base = nullptr;
  const hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return e;
  auto get_ws = [&](size_t bytes, float** out) {
    if (bytes > kGemmScratchBytes) return false;  // never: the planner keeps within it
    *out = base;
    return true;
  };
  return run_gemm(w, layout, n, k, a, m, lda, c, ldc, force.gemm_plan, static_cast<double>(kGemmScratchBytes),
                  get_ws, stream);
}

}  // namespace rfp4
