// Batch-1 GEMV on the matrix cores for tall launches (dual layout, f16 activations).
//
// What it computes is the GEMV of the dot-product kernel (gemv_impl.h): for every row,
// the sum over blocks and 16-weight halves of (half-scale x sum of codebook value x
// activation). Page "Feasibility Report: Porting ROCmFP4 to Atlas", sections "Block
// Layout" (two 16-weight halves, each with its own unsigned E4M3 scale byte),
// "Codebook10 Value Table" and "Scale Format". Only the arithmetic is arranged
// differently.
//
// Tiles of 16 rows, one per workgroup of four wavefronts. Lane l of wavefront w holds
// row l % 16 of the tile and belongs to lane group g = l / 16; it multiplies the units
// (pairs of blocks, 36 bytes) w * 4 + g, + 16, + 32, ... of its row. The units are
// loaded along rows by other lanes, three steps in flight, and handed over through LDS
// (see the kernel).
// Each 32-bit word of codes (8 weights: 4 of the first half, 4 of the second) is
// decoded on the VALU into unscaled f16 codebook values (the high-byte table of the
// dot-product kernel) and is the B fragment of one v_mfma_f32_16x16x32_f16; the eight
// words of a unit take eight MFMAs. The scales are not folded into B: the A operand
// carries the activations of each (lane group, block of the unit, half) in a row of its
// own, 4 lane groups x 2 blocks x 2 halves = 16 rows, zero elsewhere. The accumulator
// rows 4g .. 4g + 3 then hold, in the lane that loaded the unit, that unit's four half
// sums, which the lane scales with its own scale bytes. The products of the 15 other
// rows of a matrix-core pass are zero, and the MFMA adds them exactly.
//
// A rows come from LDS: per block, eight 16-byte pieces (code word d, half h) holding
// the four activations that meet that word's codes of half h in the slots where B has
// them, zeros in the other four slots; lanes whose A row is not the current (group,
// block) read a zero piece. Per 64 weights this takes ~120 VALU instructions against
// ~146 for the dot-product form (which launches it takes: gemv_tall_fits).
//
// Requirements (checked by gemv_tall_fits): dual layout, f16 activations, batch 1,
// k = 1024 * NUL with NUL in {5, 6} (the activations of a 16-lane-group split take
// NUL units per lane), every matrix's rows a multiple of 16.

#pragma once

#include "rfp4_internal.h"

namespace rfp4 {
namespace {

typedef _Float16 tall_h8 __attribute__((ext_vector_type(8)));
typedef float tall_f4 __attribute__((ext_vector_type(4)));

// High bytes of the f16 encodings of the magnitudes 0, 1, 2, 3 (low word) and 4, 6, 8,
// 10 (high word); every low byte is zero.
constexpr uint32_t kTallHiLo = 0x42403C00u;
constexpr uint32_t kTallHiHi = 0x49484644u;

// B fragment of one code word q: f16 values of the low nibbles (weights 4d .. 4d + 3 of
// the block, first half) then of the high nibbles (weights 16 + 4d .., second half).
__device__ __forceinline__ tall_h8 tall_fragment(uint32_t q) {
  const uint32_t lo =
      __builtin_amdgcn_perm(kTallHiHi, kTallHiLo, q & 0x07070707u) | ((q << 4) & 0x80808080u);
  const uint32_t hi =
      __builtin_amdgcn_perm(kTallHiHi, kTallHiLo, (q >> 4) & 0x07070707u) | (q & 0x80808080u);
  const uint32_t v[4] = {__builtin_amdgcn_perm(0u, lo, 0x010C000Cu), __builtin_amdgcn_perm(0u, lo, 0x030C020Cu),
                         __builtin_amdgcn_perm(0u, hi, 0x010C000Cu), __builtin_amdgcn_perm(0u, hi, 0x030C020Cu)};
  return __builtin_bit_cast(tall_h8, v);
}

// E4M3 value of byte BYTE of a word, sign bit ignored (the half-scale is this / 2).
template <int BYTE>
__device__ __forceinline__ float tall_scale(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word & 0x7F7F7F7Fu), BYTE);
}

struct TallUnit {
  uint32_t d[9];  // bytes 0..35 of a pair of dual blocks
};

__device__ __forceinline__ void tall_load(const uint8_t* p, TallUnit& u) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  u.d[0] = a.x; u.d[1] = a.y; u.d[2] = a.z; u.d[3] = a.w;
  u.d[4] = b.x; u.d[5] = b.y; u.d[6] = b.z; u.d[7] = b.w;
  u.d[8] = *reinterpret_cast<const uint32_t*>(p + 32);
}

// Matrices of one launch: tile t of the launch is tile t - tbeg[i] of matrix i.
struct TallParts {
  const uint8_t* w[kMaxGemvParts];
  float* y[kMaxGemvParts];
  int tbeg[kMaxGemvParts + 1];
  int count;
};

template <int NUL, bool SINGLE, bool STAGED>
__global__ __launch_bounds__(256) void gemv_tall_kernel(const TallParts parts,
                                                        const uint16_t* __restrict__ x) {
  extern __shared__ uint4 tall_xs[];  // 8 pieces per block, 8 zero pieces, the weight stage
  constexpr int kNb = 32 * NUL;       // blocks per row
  constexpr int kPieces = 8 * kNb;
  constexpr int64_t kRowBytes = 16 * NUL * 36;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  int mi = 0;
  if constexpr (!SINGLE) {
    while (mi + 1 < parts.count && static_cast<int>(blockIdx.x) >= parts.tbeg[mi + 1]) ++mi;
  }
  const int row = (static_cast<int>(blockIdx.x) - parts.tbeg[mi]) * 16 + nl;
  // STAGED: weight loads run along rows: lane l of wavefront w loads unit 16 t + l % 16
  // of tile row 4 w + l / 16 (16 consecutive units of 4 rows per load instruction, where
  // the lanes' own units span 16 rows), and each unit reaches the lane that multiplies it
  // (row l % 16, unit 16 t + 4 w + l / 16) through a double-buffered LDS stage: planes of
  // 16-byte slots (words 0-3, 4-7) and 4-byte slots (word 8) at u * 16 + (r ^ u) for row
  // r and unit u of the step, bank-conflict free for the storing and the reading lanes.
  // One barrier per step suffices: a buffer is stored again two steps later, and every
  // lane has finished reading it before it reaches the barrier in between. Otherwise each
  // lane loads the units it multiplies.
  const uint8_t* wr = STAGED ? parts.w[mi] + ((static_cast<int>(blockIdx.x) - parts.tbeg[mi]) * 16 + 4 * wv + g) * kRowBytes
                             : parts.w[mi] + row * kRowBytes;
  const int u_load = STAGED ? nl : wv * 4 + g;  // unit of each step this lane loads
  uint4* const st_a = tall_xs + kPieces + 8;  // two buffers of 256 + 256 + 64 pieces
  auto stage_put = [&](int buf, const TallUnit& u) {
    const int sl = nl * 16 + ((4 * wv + g) ^ nl);
    uint4* const b = st_a + buf * 576;
    b[sl] = uint4{u.d[0], u.d[1], u.d[2], u.d[3]};
    b[256 + sl] = uint4{u.d[4], u.d[5], u.d[6], u.d[7]};
    reinterpret_cast<uint32_t*>(b + 512)[sl] = u.d[8];
  };
  auto stage_get = [&](int buf) {
    const int un = 4 * wv + g;
    const int sl = un * 16 + (nl ^ un);
    const uint4* const b = st_a + buf * 576;
    const uint4 a = b[sl], c = b[256 + sl];
    TallUnit u;
    u.d[0] = a.x; u.d[1] = a.y; u.d[2] = a.z; u.d[3] = a.w;
    u.d[4] = c.x; u.d[5] = c.y; u.d[6] = c.z; u.d[7] = c.w;
    u.d[8] = reinterpret_cast<const uint32_t*>(b + 512)[sl];
    return u;
  };

  // Staging loads first (NUL pieces per thread), then the first weight units, then the
  // LDS stores: memory counters retire in issue order, so the stores wait for the
  // staging loads only. Piece p = (block j, code word d, half h), j = p / 8,
  // d = p / 2 % 4, h = p % 2: activations 32 j + 16 h + 4 d .. + 3 in slots 4h .. 4h + 3.
  uint2 sv[NUL];
#pragma unroll
  for (int i = 0; i < NUL; ++i) {
    const int p = threadIdx.x + 256 * i;
    sv[i] = *reinterpret_cast<const uint2*>(x + 32 * (p >> 3) + 16 * (p & 1) + 4 * ((p >> 1) & 3));
  }
  constexpr int D = 3;
  TallUnit rb[D];
#pragma unroll
  for (int t = 0; t < D; ++t) tall_load(wr + (u_load + 16 * t) * 36, rb[t]);
#pragma unroll
  for (int i = 0; i < NUL; ++i) {
    const int p = threadIdx.x + 256 * i;
    tall_xs[p] = (p & 1) ? uint4{0u, 0u, sv[i].x, sv[i].y} : uint4{sv[i].x, sv[i].y, 0u, 0u};
  }
  if (threadIdx.x < 8) tall_xs[kPieces + threadIdx.x] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();

  // This lane's A row is m = nl in k group g: it carries data iff m / 4 == g, for block
  // m / 2 % 2 and half m % 2 of its group's unit.
  const bool live = (nl >> 2) == g;
  const int bl = (nl >> 1) & 1, hl = nl & 1;
  const uint4* const zero = tall_xs + kPieces;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NUL; ++t) {
    TallUnit u;
    if constexpr (STAGED) {
      stage_put(t & 1, rb[t % D]);
      if (t + D < NUL) tall_load(wr + (u_load + 16 * (t + D)) * 36, rb[t % D]);
      __syncthreads();
      u = stage_get(t & 1);
    } else {
      u = rb[t % D];
    }
    const int un = wv * 4 + g + 16 * t;
    const uint4* a0 = (live && bl == 0) ? tall_xs + 16 * un + hl : zero;
    const uint4* a1 = (live && bl == 1) ? tall_xs + 16 * un + 8 + hl : zero;
    // The second block starts 2 bytes into word 4.
    const uint32_t q1[4] = {__builtin_amdgcn_alignbyte(u.d[5], u.d[4], 2), __builtin_amdgcn_alignbyte(u.d[6], u.d[5], 2),
                            __builtin_amdgcn_alignbyte(u.d[7], u.d[6], 2), __builtin_amdgcn_alignbyte(u.d[8], u.d[7], 2)};
    tall_f4 dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d)
      dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(tall_h8, a0[2 * d]), tall_fragment(u.d[d]), dd, 0, 0, 0);
#pragma unroll
    for (int d = 0; d < 4; ++d)
      dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(tall_h8, a1[2 * d]), tall_fragment(q1[d]), dd, 0, 0, 0);
    // Accumulator row 4g + r of this lane = (block r / 2, half r % 2) of its unit; the
    // scale bytes are bytes 16, 17 (first block) and 34, 35 (second block).
    acc[0] = __builtin_fmaf(tall_scale<0>(u.d[4]), dd[0], acc[0]);
    acc[1] = __builtin_fmaf(tall_scale<1>(u.d[4]), dd[1], acc[1]);
    acc[2] = __builtin_fmaf(tall_scale<2>(u.d[8]), dd[2], acc[2]);
    acc[3] = __builtin_fmaf(tall_scale<3>(u.d[8]), dd[3], acc[3]);
    if constexpr (!STAGED)
      if (t + D < NUL) tall_load(wr + (u_load + 16 * (t + D)) * 36, rb[t % D]);
  }
  // Sum over the four half sums, the four lane groups, then the four wavefronts (in a
  // fixed order); the 1/2 of the half-scale is applied at the store.
  float v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  __shared__ float red[4][16];
  if (g == 0) red[wv][nl] = v;
  __syncthreads();
  if (wv == 0 && g == 0) parts.y[mi][row] = 0.5f * (((red[0][nl] + red[1][nl]) + red[2][nl]) + red[3][nl]);
}

// Whether a batch-1 launch takes the tall kernel. A forced kernel (rfp4_force) turns it
// off (dot product, tiles, no-tall) or on wherever the shape allows (tall). By default,
// from timings against the dot-product kernel on one machine (tall / dot, us): fused
// launches of several matrices (gate + up 21.0 / 22.9, q + k + v 6.5 / 6.8) and single
// matrices with at least 8 tiles per CU, where the tall kernel stages its weights
// (32768 rows 19.3 / 20.8, 34816 rows 20.9 / 22.2, 69632 rows 36.8 / 39.4, 152064 rows
// 75.4 / 82.2; below that the dot-product kernel, which keeps its weight units in flight,
// was 3-8 % faster: 16384 rows 11.5 / 11.2, 24576 rows 16.1 / 14.9); k = 5120 only (at
// k = 6144 it was 7-10 % slower from 12288 rows); at least two tiles per CU, and the
// busiest CU at most 7 % above the average tile count (at 17408 rows, 4.25 tiles per CU,
// it was 2-5 % slower).
inline bool gemv_tall_fits(const GemvPart* parts, int count, int layout, int nb, int batch,
                           const Force& force) {
  if (layout != kDual || batch != 1 || (nb != 160 && nb != 192)) return false;
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    if (parts[i].n % 16 != 0) return false;
    tiles += parts[i].n / 16;
  }
  if (tiles >= (int64_t(1) << 31)) return false;
  const int fk = force.gemv_kernel;
  if (fk == RFP4_GEMV_KERNEL_DOT || fk == RFP4_GEMV_KERNEL_TILES || fk == RFP4_GEMV_KERNEL_NO_TALL) return false;
  if (fk == RFP4_GEMV_KERNEL_TALL) return true;
  if (nb != 160) return false;
  const int64_t cus = device_cu_count();
  if (count < 2 && tiles < 8 * cus) return false;
  const int64_t busiest = (tiles + cus - 1) / cus;
  return tiles >= 2 * cus && busiest * cus * 100 <= tiles * 107;
}

inline hipError_t launch_gemv_tall(const GemvPart* parts, int count, int nb, const uint16_t* x,
                                   hipStream_t stream) {
  TallParts tp;
  tp.count = count;
  tp.tbeg[0] = 0;
  for (int i = 0; i < count; ++i) {
    tp.w[i] = parts[i].w;
    tp.y[i] = parts[i].y;
    tp.tbeg[i + 1] = tp.tbeg[i] + static_cast<int>(parts[i].n / 16);
  }
  for (int i = count; i < kMaxGemvParts; ++i) {
    tp.w[i] = nullptr;
    tp.y[i] = nullptr;
    tp.tbeg[i + 1] = tp.tbeg[count];
  }
  const dim3 grid(tp.tbeg[count]), block(256);
  // The weight stage from 8 tiles per CU (measured against per-lane loads, us: fused
  // gate + up 2 x 17408 rows, 8.5 tiles per CU, 21.86 -> 20.97; 2 x 34816 rows 39.46 ->
  // 37.92; 2 x 76032 rows 81.62 -> 76.95; but 2 x 8192 rows, 4 per CU, 10.72 -> 11.26 and
  // q + k + v, 2 per CU, 6.51 -> 7.25: with few workgroups per CU its barriers are not
  // hidden).
  const bool staged = tp.tbeg[count] >= 8 * device_cu_count();
  const size_t shm = (static_cast<size_t>(nb) * 8 + 8 + (staged ? 2 * 576 : 0)) * 16;
#define RFP4_TALL_LAUNCH(NU, SG, ST) gemv_tall_kernel<NU, SG, ST><<<grid, block, shm, stream>>>(tp, x)
  if (nb == 160) {
    if (count == 1) { if (staged) RFP4_TALL_LAUNCH(5, true, true); else RFP4_TALL_LAUNCH(5, true, false); }
    else { if (staged) RFP4_TALL_LAUNCH(5, false, true); else RFP4_TALL_LAUNCH(5, false, false); }
  } else {
    if (count == 1) { if (staged) RFP4_TALL_LAUNCH(6, true, true); else RFP4_TALL_LAUNCH(6, true, false); }
    else { if (staged) RFP4_TALL_LAUNCH(6, false, true); else RFP4_TALL_LAUNCH(6, false, false); }
  }
#undef RFP4_TALL_LAUNCH
  return hipGetLastError();
}

}  // namespace
}  // namespace rfp4
