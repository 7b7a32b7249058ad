// Fused dequant + GEMV for decode: y[b][r] = sum_c W[r][c] * x[b][c], batch 1..8 (the
// dot-product kernel; larger batches default to the matrix-core kernel of gemv_mfma.h
// as use_mfma there decides).
//
// The page names gemv as the decode hot path ("Feasibility Report: Porting ROCmFP4
// to Atlas", "Kernel System" and "Integration Options", Option 2) and says that on
// AMD the bottleneck is memory bandwidth ("Why AMD is Different from NVIDIA"). The
// kernel therefore reads every packed block exactly once from HBM and does all the
// decode in registers.
//
// Loads. A lane owns units of P consecutive blocks (P = 1 or 2). A pair (P = 2) is
// 36 contiguous bytes (dual) or 34 (fast), fetched with two 16-byte loads and one
// 4-byte (dual) or 2-byte (fast) load: 1.5 memory instructions per block instead of
// 2 for single blocks (16 index bytes + a small load for the scale bytes), which
// measurably raises the achieved bandwidth. The second block of a pair starts at byte
// 18 (dual) or 17 (fast); its index bytes are realigned with v_alignbyte_b32. The
// launcher uses pairs unless that leaves too few wavefronts for the shape.
//
// Work mapping. A wavefront covers RL rows x CL lanes (RL * CL = 64); lane c of a row
// owns units c, c + CL, c + 2 CL, ... of that row (the remainder masked when CL does
// not divide the units of a row), so each load instruction reads runs of CL * 36 (or
// 34, 18, 17) contiguous bytes. The grid is a whole number r of workgroups per CU, all
// resident (the LDS request pins r), and workgroup w owns an equal contiguous share of
// the row groups, which its wavefronts take round-robin: every CU gets the same work.
// Each lane keeps two or three units in flight (depth_for), with every load issued
// unconditionally so that the compiler's waits count exactly the units behind the one
// consumed.
//
// Arithmetic. Each block's 32 weights are decoded to f16/bf16 pairs of unscaled codebook
// values (f16: high-byte table plus zero-spread, below; bf16: E4M3 codes and the packed
// FP8 conversion of rfp4_decode.h) and multiplied with the activations with
// v_dot2_f32_{f16,bf16}: one fp32 partial sum per 16-weight half, then one fp32 FMA with
// that half's E4M3 scale. The partial sums of the CL lanes of a row are combined with DPP
// additions and a swizzle (row_sum) and the 1/2 of the half-scale is applied at the store.
//
// Activations are staged once per workgroup into LDS when they fit the budget (layout
// at xs_index), with the first staging loads issued ahead of the first weight units;
// otherwise they are read from global memory, where they stay cache-resident.

#pragma once

#include "rfp4_decode.h"
#include "rfp4_internal.h"

namespace rfp4 {
namespace {

// Workgroups of 256 threads, or 1024 when long activation rows are staged in LDS (the
// staging is then shared by 16 wavefronts and two workgroups fit a CU).
#ifndef RFP4_GEMV_SMALL_THREADS
#define RFP4_GEMV_SMALL_THREADS 256
#endif
constexpr int kThreadsSmall = RFP4_GEMV_SMALL_THREADS;
constexpr int kThreadsLarge = 1024;
constexpr int kXLdsBudget = 40 * 1024;
constexpr int kXLdsBudgetLarge = 80 * 1024;

// Tuning knob (no effect on results): resident wavefronts per CU the launch is sized for.
#ifndef RFP4_GEMV_WAVES_PER_CU
#define RFP4_GEMV_WAVES_PER_CU 24
#endif

template <int XT>
struct Act;

template <>
struct Act<kF16> {
  typedef f16x2 pair;
  static __device__ __forceinline__ pair decode(uint32_t codes, bool hi) { return pair_f16(codes, hi); }
  static __device__ __forceinline__ float dot(pair w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2(w, __builtin_bit_cast(f16x2, x), acc, false);
  }
};

template <>
struct Act<kBF16> {
  typedef bf16x2 pair;
  static __device__ __forceinline__ pair decode(uint32_t codes, bool hi) { return pair_bf16(codes, hi); }
  static __device__ __forceinline__ float dot(pair w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2, x), acc, false);
  }
};

// High bytes of the f16 encodings of the magnitudes 0, 1, 2, 3 (low word, byte 0
// first) and 4, 6, 8, 10 (high word); the low bytes are all zero.
constexpr uint32_t kF16HiLo = 0x42403C00u;
constexpr uint32_t kF16HiHi = 0x49484644u;

// Four f16 high bytes (byte i = weight of the low / high nibble of byte i of q).
__device__ __forceinline__ uint32_t f16_high_bytes_low(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kF16HiHi, kF16HiLo, q & 0x07070707u);
  return mag | ((q << 4) & 0x80808080u);
}

__device__ __forceinline__ uint32_t f16_high_bytes_high(uint32_t q) {
  const uint32_t mag = __builtin_amdgcn_perm(kF16HiHi, kF16HiLo, (q >> 4) & 0x07070707u);
  return mag | (q & 0x80808080u);
}

// f16 pair of weights 0, 1 (or 2, 3) from four high bytes: selector 0x0C gives a zero byte.
__device__ __forceinline__ f16x2 spread_f16(uint32_t h, bool hi_pair) {
  const uint32_t v = __builtin_amdgcn_perm(0u, h, hi_pair ? 0x030C020Cu : 0x010C000Cu);
  return __builtin_bit_cast(f16x2, v);
}

// Weight loads (each weight byte is read once per launch). RFP4_GEMV_NT_LOADS selects
// non-temporal loads (tuning knob, no effect on results); measured slower (up-projection
// 12.5 -> 16.6 us): the loads of a unit share cache lines, which then are not kept.
#ifndef RFP4_GEMV_NT_LOADS
#define RFP4_GEMV_NT_LOADS 0
#endif
typedef uint32_t wu4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 wload16(const void* p) {
#if RFP4_GEMV_NT_LOADS
  const wu4 v = __builtin_nontemporal_load(static_cast<const wu4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
#else
  return *static_cast<const uint4*>(p);
#endif
}
__device__ __forceinline__ uint32_t wload4(const void* p) {
#if RFP4_GEMV_NT_LOADS
  return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
#else
  return *static_cast<const uint32_t*>(p);
#endif
}

// Raw bytes of one unit of P consecutive blocks (see the file comment), as words.
// Once realigned (unit_aligned):
//   P = 1: d[0..3] = index bytes, d[4] = the scale byte(s) in its low bytes.
//   P = 2: d[0..7] = bytes 0..31, d[8] = bytes 32..35 (dual) or 32..33 (fast).
// A unit of a realigned kind (below) holds, between its load and its use, the words
// from the word boundary below its first byte, and sh = that byte's offset in the word.
template <int P>
struct UnitRaw {
  uint32_t d[P == 1 ? 5 : 9];
  uint32_t sh;
};

// Units whose size is not a multiple of 4 bytes (single blocks; pairs of 17-byte
// blocks) start at 1-, 2- or 3-byte offsets. Such a unit is read with dword-aligned
// loads from the word boundary below it and shifted into place per lane with
// v_alignbyte_b32: unaligned 16-byte loads cost the memory pipeline measurably more.
// The extra bytes read lie in the last word that holds a byte of the unit (dual units
// and pairs of fast blocks start at even offsets, since their rows hold an even number
// of bytes), so a read never reaches past the word of the matrix's last byte and never
// crosses into another page.
template <int LAYOUT, int P>
constexpr bool unit_realigned() {
  return (P * block_bytes(LAYOUT)) % 4 != 0 || P == 1;
}

// The shift is applied where the unit is used (unit_aligned), not here: the loaded
// words must not be touched until the unit is due, or the compiler waits for this
// load at once and the units meant to be in flight behind it never are.
template <int LAYOUT, int P>
__device__ __forceinline__ void load_unit_realigned(const uint8_t* p, UnitRaw<P>& u) {
  constexpr int NW = P == 1 ? 5 : 9;  // words covering the unit from its word boundary
  const uint32_t sh = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);
  const uint32_t* a = reinterpret_cast<const uint32_t*>(p - sh);
  const uint4 v0 = wload16(a);
  u.d[0] = v0.x;
  u.d[1] = v0.y;
  u.d[2] = v0.z;
  u.d[3] = v0.w;
  if constexpr (P == 2) {
    const uint4 v1 = wload16(a + 4);
    u.d[4] = v1.x;
    u.d[5] = v1.y;
    u.d[6] = v1.z;
    u.d[7] = v1.w;
  }
  u.d[NW - 1] = wload4(a + NW - 1);
  u.sh = sh;
}

// The unit's words realigned to its first byte (a copy for the layouts loaded aligned).
template <int LAYOUT, int P>
__device__ __forceinline__ UnitRaw<P> unit_aligned(const UnitRaw<P>& r) {
  if constexpr (unit_realigned<LAYOUT, P>()) {
    constexpr int NW = P == 1 ? 5 : 9;
    UnitRaw<P> u;
#pragma unroll
    for (int i = 0; i < NW - 1; ++i) u.d[i] = __builtin_amdgcn_alignbyte(r.d[i + 1], r.d[i], r.sh);
    u.d[NW - 1] = r.d[NW - 1] >> (8 * r.sh);
    u.sh = 0;
    return u;
  } else {
    return r;
  }
}

template <int LAYOUT, int P>
__device__ __forceinline__ void load_unit(const uint8_t* p, UnitRaw<P>& u) {
  if constexpr (unit_realigned<LAYOUT, P>()) {
    load_unit_realigned<LAYOUT, P>(p, u);
    return;
  }
  u.sh = 0;
  const uint4 v0 = wload16(p);
  u.d[0] = v0.x;
  u.d[1] = v0.y;
  u.d[2] = v0.z;
  u.d[3] = v0.w;
  if constexpr (P == 1) {
    if constexpr (LAYOUT == kDual) {
      uint16_t t;
      __builtin_memcpy(&t, p + 16, 2);
      u.d[4] = t;
    } else {
      u.d[4] = p[16];
    }
  } else {
    const uint4 v1 = wload16(p + 16);
    u.d[4] = v1.x;
    u.d[5] = v1.y;
    u.d[6] = v1.z;
    u.d[7] = v1.w;
    if constexpr (LAYOUT == kDual) {
      u.d[8] = wload4(p + 32);  // 4-byte aligned: units start at multiples of 36 bytes
                               // (P = 2 needs an even block count, so rows hold 36j bytes)
    } else {
      uint16_t t;
      __builtin_memcpy(&t, p + 32, 2);
      u.d[8] = t;
    }
  }
}

// The 16 index bytes of block B of a unit, as four words.
template <int LAYOUT, int P, int B>
__device__ __forceinline__ uint4 unit_qs(const UnitRaw<P>& u) {
  constexpr int off = B * block_bytes(LAYOUT);  // byte offset of the block in the unit
  constexpr int w0 = off / 4;
  constexpr int sh = off % 4;
  if constexpr (sh == 0) {
    return uint4{u.d[w0], u.d[w0 + 1], u.d[w0 + 2], u.d[w0 + 3]};
  } else {
    return uint4{__builtin_amdgcn_alignbyte(u.d[w0 + 1], u.d[w0], sh),
                 __builtin_amdgcn_alignbyte(u.d[w0 + 2], u.d[w0 + 1], sh),
                 __builtin_amdgcn_alignbyte(u.d[w0 + 3], u.d[w0 + 2], sh),
                 __builtin_amdgcn_alignbyte(u.d[w0 + 4], u.d[w0 + 3], sh)};
  }
}

// E4M3 values of the scale byte(s) of block B (twice the decoded scales). Bit 7 of a
// scale byte is not part of the value and is cleared first.
template <int LAYOUT, int P, int B>
__device__ __forceinline__ void unit_scales(const UnitRaw<P>& u, float& s0, float& s1) {
  constexpr int off = (P == 1) ? 0 : B * block_bytes(LAYOUT) + 16;
  constexpr int wi = (P == 1) ? 4 : off / 4;
  constexpr int bi = off % 4;
  const uint32_t word = u.d[wi] & 0x7F7F7F7Fu;
  s0 = e4m3_hw<bi>(word);
  if constexpr (LAYOUT == kDual) {
    static_assert(bi == 0 || bi == 2, "dual scale bytes are 2-byte aligned");
    s1 = e4m3_hw<bi + 1>(word);
  } else {
    s1 = s0;
  }
}

// One block: decode 32 weights and accumulate them against every activation row.
// `xunit(b, cc)` returns the 16-byte activation unit cc (values 8cc..8cc+7 of the
// block) of activation row b.
template <int XT, int BATCH, typename XUnit>
__device__ __forceinline__ void block_dot(uint4 qv, float s0, float s1, bool valid, XUnit xunit,
                                          float (&acc)[BATCH]) {
  typedef Act<XT> A;
  typedef typename A::pair pair;
  const uint32_t q[4] = {qv.x, qv.y, qv.z, qv.w};
  pair wl[8], wh[8];  // first half (low nibbles), second half (high nibbles)
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (XT == kF16) {
      // Every codebook magnitude is an f16 value whose low byte is zero: look up the
      // high bytes (sign in bit 7) and spread them into f16 pairs with zero low bytes.
      const uint32_t lo = f16_high_bytes_low(q[d]);
      const uint32_t hi = f16_high_bytes_high(q[d]);
      wl[2 * d] = spread_f16(lo, false);
      wl[2 * d + 1] = spread_f16(lo, true);
      wh[2 * d] = spread_f16(hi, false);
      wh[2 * d + 1] = spread_f16(hi, true);
    } else {
      const uint32_t lo = codes_low(q[d]);
      const uint32_t hi = codes_high(q[d]);
      wl[2 * d] = A::decode(lo, false);
      wl[2 * d + 1] = A::decode(lo, true);
      wh[2 * d] = A::decode(hi, false);
      wh[2 * d + 1] = A::decode(hi, true);
    }
  }
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    uint4 xc[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) xc[cc] = xunit(b, cc);
    const uint32_t x0[8] = {xc[0].x, xc[0].y, xc[0].z, xc[0].w, xc[1].x, xc[1].y, xc[1].z, xc[1].w};
    const uint32_t x1[8] = {xc[2].x, xc[2].y, xc[2].z, xc[2].w, xc[3].x, xc[3].y, xc[3].z, xc[3].w};
    // One fp32 chain per 16-weight half (two chains per half, joined at the end,
    // measured 1-4 % slower on most decode shapes: two more instructions per block).
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      p0 = A::dot(wl[t], x0[t], p0);
      p1 = A::dot(wh[t], x1[t], p1);
    }
    // A masked lane adds nothing: its products may be 0 * inf = NaN, so they are
    // dropped, not scaled by zero.
    acc[b] = __builtin_fmaf(s0, valid ? p0 : 0.f, acc[b]);
    acc[b] = __builtin_fmaf(s1, valid ? p1 : 0.f, acc[b]);
  }
}

// Sum over the CL = 2^log2cl consecutive lanes of a row, left in every one of them
// (the same bits in each, since every step adds two equally ordered partial sums): DPP
// within 16-lane rows (quad_perm swaps of neighbours and of pairs, then the half-row and
// row mirrors, which pair each lane with one of the other quad or half once those hold
// equal sums), then a swizzle that exchanges 16-lane rows (xor 16) and, for 64 lanes per
// row, a shuffle across the halves of the wavefront. The 16-lane steps need no LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum(float v, int log2cl) {
  if (log2cl >= 1) v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if (log2cl >= 2) v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if (log2cl >= 3) v = dpp_add<0x141>(v);  // row_half_mirror
  if (log2cl >= 4) v = dpp_add<0x140>(v);  // row_mirror
  // ds_swizzle bit mode: and-mask 0x1F, or-mask 0, xor-mask 0x10 (within 32 lanes)
  if (log2cl >= 5)
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if (log2cl >= 6) v += __shfl_xor(v, 32, 64);
  return v;
}

// Activation layout in LDS: for activation row b and unit column ud (blocks P*ud ..
// P*ud + P - 1), 4P consecutive 16-byte units (block-major, then 8-value chunk) plus
// one padding unit, so a lane reads all of its unit's activations from one base
// address with immediate offsets, and the lanes of a row (consecutive ud, stride
// (4P+1)*16 bytes) hit distinct banks.
template <int P>
__device__ __forceinline__ int xs_index(int b, int ud, int nu, int B, int cc) {
  return (b * nu + ud) * (4 * P + 1) + 4 * B + cc;
}

// `xu` points at the lane's first activation unit for this block column (row b = 0):
// LDS unit (ud * (4P+1)) when XLDS, else the global address of block P*ud.
template <int LAYOUT, int XT, int BATCH, bool XLDS, int P, int B>
__device__ __forceinline__ void unit_block(const UnitRaw<P>& u, const uint4* xu, int xrow,
                                           const uint16_t* xg, int64_t ldx, bool valid,
                                           float (&acc)[BATCH]) {
  float s0, s1;
  unit_scales<LAYOUT, P, B>(u, s0, s1);
  // A lane past the end of a ragged row re-reads the row's last unit (weights and
  // activations); block_dot drops its contribution.
  auto xunit = [&](int b, int cc) -> uint4 {
    if constexpr (XLDS)
      return xu[b * xrow + 4 * B + cc];
    else
      return *reinterpret_cast<const uint4*>(xg + b * ldx + 32 * B + 8 * cc);
  };
  block_dot<XT, BATCH>(unit_qs<LAYOUT, P, B>(u), s0, s1, valid, xunit, acc);
}

// The matrices of one launch (up to kMaxGemvParts, sharing k and the activations):
// part i has n[i] rows at w[i], outputs at y[i] with leading dimension ldy[i], and
// owns row groups [gbeg[i], gbeg[i + 1]) of the launch.
// Single-matrix launches use NP = 1: a small argument block that every wavefront reads
// at start (the eight-entry block measurably slows short launches).
template <int NP>
struct GemvParts {
  const uint8_t* w[NP];
  float* y[NP];
  int64_t ldy[NP];
  int n[NP];
  int gbeg[NP + 1];
  int count;
};

template <int LAYOUT, int XT, int BATCH, bool XLDS, int P, bool RAGGED, int THREADS, int NP, int D>
__global__ __launch_bounds__(THREADS) void gemv_kernel(const GemvParts<NP> parts, int nu, int log2cl,
                                                        int groups,
                                                        const uint16_t* __restrict__ x,
                                                        int64_t ldx) {
  constexpr int UB = P * block_bytes(LAYOUT);  // bytes per unit
  extern __shared__ uint4 xs[];

  const int lane = threadIdx.x & 63;
  const int cl = 1 << log2cl;
  const int rl = 64 >> log2cl;
  const int r_in = lane >> log2cl;
  const int c = lane & (cl - 1);
  // Units per lane per row. When CL does not divide the units of a row (RAGGED), the
  // last iteration covers the remainder and the lanes past the end are masked.
  const int iters = RAGGED ? (nu + cl - 1) >> log2cl : nu >> log2cl;
  // readfirstlane tells the compiler the wavefront index is uniform, so every cursor
  // and loop bound derived from it lives in scalar registers.
  // Workgroup w owns the row groups [G w / WGs, G (w + 1) / WGs): the grid is a whole
  // number of workgroups per CU, all resident, so every CU gets the same share (to one
  // group). Its wavefronts take the groups round-robin.
  constexpr int S = THREADS / 64;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g0 = static_cast<int>(static_cast<int64_t>(groups) * blockIdx.x / gridDim.x);
  const int g1 = static_cast<int>(static_cast<int64_t>(groups) * (blockIdx.x + 1) / gridDim.x);
  const int g_begin = g0 + wv;
  const int my_groups = g1 > g_begin ? (g1 - g_begin + S - 1) / S : 0;
  const int total = my_groups * iters;  // units per lane
  const int64_t rowbytes = static_cast<int64_t>(nu) * UB;  // < 2^31 / 64 (checked by the launcher)

  // Load cursor over (row group, unit index); wave-uniform. The address of the next
  // unit is kept as a wave-uniform part (row group base + unit offset) plus a per-lane
  // offset (row within the group, clamped to the last row, and lane column), so
  // advancing the cursor costs scalar additions only.
  // The groups of the launch are those of the parts (matrices) one after another; a
  // cursor moving forward finds its part by advancing a part index.
  // A launch of one matrix (the common case) takes a path without part lookups.
  constexpr bool single = NP == 1;
  const uint8_t* const w0 = parts.w[0];
  const int n0 = parts.n[0];
  auto part_of = [&](int g, int& mi) {
    if (!single)
      while (mi + 1 < parts.count && g >= parts.gbeg[mi + 1]) ++mi;
  };
  int li = 0, issued = 0;
  const int64_t group_stride = static_cast<int64_t>(rl) * rowbytes;
  const int unit_stride = cl * UB;
  const int c_off = c * UB;
  const int last_off = (nu - 1) * UB;
  int lg = g_begin;
  int mi_l = 0;
  const uint8_t* gbase = nullptr;
  int lane_off = 0;
  auto seek = [&]() {  // base of group lg; rows past the part's end clamp to its last row
    if (single) {
      gbase = w0 + static_cast<int64_t>(lg) * group_stride;
      lane_off = min(r_in, max(n0 - 1 - lg * rl, 0)) * static_cast<int>(rowbytes);
    } else {
      part_of(lg, mi_l);
      const int gl = lg - parts.gbeg[mi_l];
      gbase = parts.w[mi_l] + static_cast<int64_t>(gl) * group_stride;
      lane_off = min(r_in, max(parts.n[mi_l] - 1 - gl * rl, 0)) * static_cast<int>(rowbytes);
    }
  };
  seek();
  int unit_off = 0;
  auto advance = [&]() {
    ++issued;
    unit_off += unit_stride;
    if (++li == iters) {
      li = 0;
      unit_off = 0;
      lg += S;
      if (single) {
        gbase += S * group_stride;
        lane_off = min(r_in, max(n0 - 1 - lg * rl, 0)) * static_cast<int>(rowbytes);
      } else if (issued < total) {
        seek();
      }
    }
  };
  // Every load is issued unconditionally (straight-line loads let the compiler wait for
  // exactly the loads it needs; a load skipped on some path makes its waits count that
  // path, draining every load in flight): a wavefront with no unit left loads the first
  // unit of the launch instead (in bounds, one cache line) and never consumes it.
  auto load_next = [&](UnitRaw<P>& buf) {
    const bool live = issued < total;  // wave-uniform
    const int col = RAGGED ? min(unit_off + c_off, last_off) : unit_off + c_off;
    load_unit<LAYOUT, P>(live ? gbase + static_cast<uint32_t>(col + lane_off) : w0, buf);
    if (live) advance();
  };

  // D units in flight per lane (depth_for). With the activations staged in LDS, the
  // first staging loads are issued before the weight units, so the LDS stores wait only
  // for them (memory counters retire in issue order) while the weight loads stay in
  // flight; each consumed unit is then replaced by the next one.
  UnitRaw<P> rb[D];
  if constexpr (XLDS) {
    const int units = BATCH * 4 * nu * P;  // 16-byte activation units
    auto src_of = [&](int t) {  // global address of activation unit t
      const int cc = t & 3;
      const int jb = t >> 2;  // block index over all activation rows
      const int b = BATCH == 1 ? 0 : jb / (nu * P);
      const int j = jb - b * nu * P;
      return reinterpret_cast<const uint4*>(x + b * ldx + 32 * j + 8 * cc);
    };
    auto dst_of = [&](int t) {
      const int cc = t & 3;
      const int jb = t >> 2;
      const int b = BATCH == 1 ? 0 : jb / (nu * P);
      const int j = jb - b * nu * P;
      return xs + xs_index<P>(b, j / P, nu, j % P, cc);
    };
    // Four chunks per thread and round; the loads are clamped, so every lane loads in
    // bounds, and only the stores are masked.
    auto stage = [&](int t0, bool first) {
      const uint4 v0 = *src_of(min(t0, units - 1));
      const uint4 v1 = *src_of(min(t0 + THREADS, units - 1));
      const uint4 v2 = *src_of(min(t0 + 2 * THREADS, units - 1));
      const uint4 v3 = *src_of(min(t0 + 3 * THREADS, units - 1));
      if (first) {  // uniform: the first round of every thread
#pragma unroll
        for (int d = 0; d < D; ++d) load_next(rb[d]);
      }
      if (t0 < units) *dst_of(t0) = v0;
      if (t0 + THREADS < units) *dst_of(t0 + THREADS) = v1;
      if (t0 + 2 * THREADS < units) *dst_of(t0 + 2 * THREADS) = v2;
      if (t0 + 3 * THREADS < units) *dst_of(t0 + 3 * THREADS) = v3;
    };
    stage(threadIdx.x, true);
    for (int t0 = threadIdx.x + 4 * THREADS; t0 < units; t0 += 4 * THREADS) stage(t0, false);
    __syncthreads();
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) load_next(rb[d]);
  }

  float acc[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) acc[b] = 0.f;

  // Compute cursor; wave-uniform. Activation pointers advance by whole unit columns.
  int cg = g_begin, ci = 0, mi_c = 0;
  part_of(cg, mi_c);
  const int xrow = nu * (4 * P + 1);  // LDS units per activation row
  const uint4* xu0 = xs + c * (4 * P + 1);
  const uint16_t* xg0 = x + 32 * P * c;
  auto consume = [&](const UnitRaw<P>& u) {
    const int row = (single ? cg : cg - parts.gbeg[mi_c]) * rl + r_in;
    const int uidx = c + ci * cl;  // unit of the row this lane holds
    const bool valid = !RAGGED || uidx < nu;
    const int ux = RAGGED ? min(uidx, nu - 1) : uidx;
    const uint4* xu = RAGGED ? xs + ux * (4 * P + 1) : xu0 + ci * (cl * (4 * P + 1));
    const uint16_t* xg = RAGGED ? x + 32 * P * ux : xg0 + ci * (32 * P * cl);
    // Rows past n were loaded from a clamped address; their sums are never stored.
    const UnitRaw<P> ua = unit_aligned<LAYOUT, P>(u);
    unit_block<LAYOUT, XT, BATCH, XLDS, P, 0>(ua, xu, xrow, xg, ldx, valid, acc);
    if constexpr (P == 2) unit_block<LAYOUT, XT, BATCH, XLDS, P, 1>(ua, xu, xrow, xg, ldx, valid, acc);
    if (++ci == iters) {  // row group complete: reduce over the CL lanes of each row
#pragma unroll
      for (int b = 0; b < BATCH; ++b) acc[b] = row_sum(acc[b], log2cl);
      if (c == 0 && row < (single ? n0 : parts.n[mi_c])) {
        float* y = single ? parts.y[0] : parts.y[mi_c];
        const int64_t ldy = single ? parts.ldy[0] : parts.ldy[mi_c];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) y[b * ldy + row] = 0.5f * acc[b];
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) acc[b] = 0.f;
      ci = 0;
      cg += S;
      part_of(cg, mi_c);
    }
  };

  // Rounds of D units: while another round follows, each consumed unit is replaced by
  // a load (of the next unit, or of the launch's first unit once none is left); the
  // last round loads nothing, so no load outlives the last unit.
  int t = 0;
  for (; t + D < total; t += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      consume(rb[d]);
      load_next(rb[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (t + d < total) consume(rb[d]);
}


struct Plan {
  int p, nu, log2cl, groups, wgs, threads, waves;
  bool ragged;
};

// Row groups of RL rows over all parts (a group never spans two parts).
inline int count_groups(const GemvPart* parts, int count, int rl) {
  int64_t g = 0;
  for (int i = 0; i < count; ++i) g += (parts[i].n + rl - 1) / rl;
  return static_cast<int>(g);
}

// Work plan for P consecutive blocks per lane unit and CL = 2^log2cl lanes per row:
// `waves` = wavefronts that get at least one row group when the grid is wgs =
// CUs * r workgroups.
inline Plan make_plan(int p, int log2cl, const GemvPart* parts, int count, int nb,
                      int waves_per_cu, int threads) {
  Plan pl;
  pl.p = p;
  pl.nu = nb / p;
  pl.log2cl = log2cl;
  pl.threads = threads;
  const int cl = 1 << log2cl;
  pl.ragged = (pl.nu % cl) != 0;
  const int rl = 64 >> log2cl;
  pl.groups = count_groups(parts, count, rl);
  // r workgroups per CU: as many as the row groups fill (every wavefront busy), at most
  // what the occupancy target allows.
  const int per_wg = threads / 64;
  const int cus = device_cu_count();
  const int r_max = waves_per_cu / per_wg > 0 ? waves_per_cu / per_wg : 1;
  const int64_t slots = static_cast<int64_t>(cus) * per_wg;
  int r = static_cast<int>((pl.groups + slots - 1) / slots);
  r = r < 1 ? 1 : (r > r_max ? r_max : r);
  pl.wgs = cus * r;
  pl.waves = pl.groups < pl.wgs * per_wg ? pl.groups : pl.wgs * per_wg;
  return pl;
}

// Lane mapping, from a sweep of all mappings on the decode shapes (17408 x 5120,
// 6144 x 5120, 1024 x 5120, 5120 x 6144, 5120 x 17408): with the activations in LDS,
// pairs of blocks per unit (fewer load instructions) and the fewest lanes per row that
// still give >= 8 busy wavefronts per CU (CL = gcd(64, units per row) or more, with
// the remainder masked); with activations read from global memory (long rows), single
// blocks and 64 lanes per row. A forced mapping (rfp4_force: P blocks per unit, CL
// lanes per row) replaces the choice; a pair mapping on an odd block count is ignored.
inline Plan choose_plan(const GemvPart* parts, int count, int nb, int waves_per_cu, bool xlds,
                        int threads, const Force& force) {
  const int fp = force.gemv_unit_blocks, fcl = force.gemv_lanes_per_row;
  if (fp != 0 && (fp == 1 || nb % 2 == 0)) {
    int l = 0;
    while ((1 << l) < fcl) ++l;
    return make_plan(fp, l, parts, count, nb, waves_per_cu, threads);
  }
  const int p = (xlds && nb % 2 == 0) ? 2 : 1;
  if (!xlds) return make_plan(1, 6, parts, count, nb, waves_per_cu, threads);
  const int nu = nb / p;
  int g = 64;
  while (nu % g) g >>= 1;  // gcd(64, nu)
  int l = 0;
  while ((1 << l) < g) ++l;
  const int want = 8 * device_cu_count();
  Plan pl = make_plan(p, l, parts, count, nb, waves_per_cu, threads);
  while (l < 6 && pl.waves < want) {
    ++l;
    pl = make_plan(p, l, parts, count, nb, waves_per_cu, threads);
  }
  return pl;
}

// Weight units in flight per lane. Every load is issued unconditionally (see the
// kernel), so a lane whose units do not fill its last round of D loads the launch's
// first unit in their place: depth 3 when the busiest lane has exactly three units (all
// issued up front, none repeated), else 2. Measured against depth 3 everywhere (one box,
// outputs bitwise equal): up-projection 12.55 -> 12.06 us, batch 2 16.55 -> 16.02;
// 5120 x 17408 fast bf16 batch 1/2 14.78/17.92 -> 14.21/17.41; 5120 x 17408 dual f16
// 14.66 -> 13.79; while 6144 x 5120 (three units per lane) takes 6.50 us at depth 3 and
// 6.70 at 2. Batches above 2 (on this kernel only when forced) keep depth 3.
inline int depth_for(const Plan& pl, int batch) {
  if (batch > 2) return 3;
  const int per_wg = pl.threads / 64;
  const int groups_wg = (pl.groups + pl.wgs - 1) / pl.wgs;  // largest workgroup share
  const int groups_wave = (groups_wg + per_wg - 1) / per_wg;
  const int iters = (pl.nu + (1 << pl.log2cl) - 1) >> pl.log2cl;
  return static_cast<int64_t>(groups_wave) * iters == 3 ? 3 : 2;
}

// The 1024-thread kernels may need more than 64 KB of dynamic LDS; the limit is raised
// once per process for each P (an idempotent call, so threads that race repeat it
// harmlessly).
template <int LAYOUT, int XT, int BATCH, int NP, int D>
hipError_t raise_lds_limit(int p) {
  static std::atomic<bool> done[2];
  std::atomic<bool>& d = done[p - 1];
  if (d.load(std::memory_order_acquire)) return hipSuccess;
  const void* fns[2] = {
      reinterpret_cast<const void*>(p == 2 ? &gemv_kernel<LAYOUT, XT, BATCH, true, 2, false, kThreadsLarge, NP, D>
                                           : &gemv_kernel<LAYOUT, XT, BATCH, true, 1, false, kThreadsLarge, NP, D>),
      reinterpret_cast<const void*>(p == 2 ? &gemv_kernel<LAYOUT, XT, BATCH, true, 2, true, kThreadsLarge, NP, D>
                                           : &gemv_kernel<LAYOUT, XT, BATCH, true, 1, true, kThreadsLarge, NP, D>)};
  for (const void* f : fns) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
  }
  d.store(true, std::memory_order_release);
  return hipSuccess;
}

template <int LAYOUT, int XT, int BATCH, int NP>
hipError_t launch3(const GemvPart* parts, int count, int nb, const uint16_t* x, int64_t ldx,
                   const Force& force, hipStream_t stream) {
  // Activation bytes in LDS (largest unit size: 4P+1 units of 16 bytes per P blocks).
  // Long rows are staged in the layout of the units the plan uses: pairs of blocks (9
  // chunks per 2 blocks) when the block count is even, else single blocks (5 per block).
  const size_t xbytes1 = static_cast<size_t>(BATCH) * nb * 5 * 16;
  const size_t xbytes2 = static_cast<size_t>(BATCH) * (nb / 2) * 9 * 16;
  const size_t xbytes_large = nb % 2 == 0 ? xbytes2 : xbytes1;
  const bool small_x = xbytes1 <= static_cast<size_t>(kXLdsBudget);
  const bool large_x = !small_x && xbytes_large <= static_cast<size_t>(kXLdsBudgetLarge);
  const bool xlds = small_x || large_x;
  const int threads = large_x ? kThreadsLarge : kThreadsSmall;
  const size_t xbytes_fit = large_x ? xbytes_large : xbytes1;
  // Resident wavefronts per CU: the knob (two whole 16-wavefront workgroups for long
  // rows), capped by what LDS allows (160 KB per CU).
  int waves_per_cu = large_x ? 2 * (kThreadsLarge / 64) : RFP4_GEMV_WAVES_PER_CU;
  if (xlds) {
    const int wg_fit = static_cast<int>((160 * 1024) / xbytes_fit);
    if (wg_fit * (threads / 64) < waves_per_cu) waves_per_cu = wg_fit * (threads / 64);
  }
  Plan pl = choose_plan(parts, count, nb, waves_per_cu, xlds, threads, force);
  // A forced single-block mapping whose staging layout would not fit takes pairs.
  if (large_x && pl.p == 1 && xbytes1 > static_cast<size_t>(kXLdsBudgetLarge))
    pl = make_plan(2, pl.log2cl, parts, count, nb, waves_per_cu, threads);
  // Activations from global memory: single blocks per unit (a forced P = 2 mapping keeps
  // its lane count).
  if (!xlds && pl.p == 2) pl = make_plan(1, pl.log2cl, parts, count, nb, waves_per_cu, threads);
  // Per-lane row offsets are 32-bit: a forced mapping with several rows per wavefront
  // falls back to one row per wavefront when the rows are too long for them.
  if (static_cast<int64_t>((64 >> pl.log2cl) - 1) * nb * block_bytes(LAYOUT) >= (int64_t(1) << 31))
    pl = make_plan(1, 6, parts, count, nb, waves_per_cu, threads);
  GemvParts<NP> gp;
  gp.count = count;
  gp.gbeg[0] = 0;
  const int rl = 64 >> pl.log2cl;
  for (int i = 0; i < count; ++i) {
    gp.w[i] = parts[i].w;
    gp.y[i] = parts[i].y;
    gp.ldy[i] = parts[i].ldy;
    gp.n[i] = static_cast<int>(parts[i].n);
    gp.gbeg[i + 1] = gp.gbeg[i] + static_cast<int>((parts[i].n + rl - 1) / rl);
  }
  const dim3 grid(pl.wgs), block(pl.threads);
  // Dynamic LDS: the staged activations, raised to just over 1 / (r + 1) of the CU's
  // 160 KB so that exactly r = wgs / CUs workgroups are resident per CU (the even split
  // of row groups relies on it).
  const int r = pl.wgs / device_cu_count();
  const size_t pin = (160 * 1024) / (r + 1) + 1024;
  size_t shm = xlds ? (pl.p == 2 ? xbytes2 : xbytes1) : 0;
  if (shm < pin) shm = pin;
  // Depth 2 exists for batches 1 and 2 only (kD2 is 3 otherwise, so no other kernel is
  // instantiated).
  constexpr int kD2 = BATCH <= 2 ? 2 : 3;
  const bool d2 = depth_for(pl, BATCH) == 2;
  if (large_x && shm > 64 * 1024) {
    const hipError_t e = d2 ? raise_lds_limit<LAYOUT, XT, BATCH, NP, kD2>(pl.p)
                            : raise_lds_limit<LAYOUT, XT, BATCH, NP, 3>(pl.p);
    if (e != hipSuccess) return e;
  }
#define RFP4_GEMV_LAUNCH(XL, PP, RG, TH)                                                     \
  do {                                                                                       \
    if (d2)                                                                                  \
      gemv_kernel<LAYOUT, XT, BATCH, XL, PP, RG, TH, NP, kD2><<<grid, block, shm, stream>>>( \
          gp, pl.nu, pl.log2cl, pl.groups, x, ldx);                                          \
    else                                                                                     \
      gemv_kernel<LAYOUT, XT, BATCH, XL, PP, RG, TH, NP, 3><<<grid, block, shm, stream>>>(   \
          gp, pl.nu, pl.log2cl, pl.groups, x, ldx);                                          \
  } while (0)
#define RFP4_GEMV_LAUNCH_P(XL, RG, TH) \
  if (pl.p == 2) RFP4_GEMV_LAUNCH(XL, 2, RG, TH); else RFP4_GEMV_LAUNCH(XL, 1, RG, TH)
  if (large_x) {
    if (pl.ragged) { RFP4_GEMV_LAUNCH_P(true, true, kThreadsLarge); } else { RFP4_GEMV_LAUNCH_P(true, false, kThreadsLarge); }
  } else if (xlds) {
    if (pl.ragged) { RFP4_GEMV_LAUNCH_P(true, true, kThreadsSmall); } else { RFP4_GEMV_LAUNCH_P(true, false, kThreadsSmall); }
  } else {
    if (pl.ragged) { RFP4_GEMV_LAUNCH(false, 1, true, kThreadsSmall); } else { RFP4_GEMV_LAUNCH(false, 1, false, kThreadsSmall); }
  }
#undef RFP4_GEMV_LAUNCH_P
#undef RFP4_GEMV_LAUNCH
  return hipGetLastError();
}

template <int LAYOUT, int XT, int NP>
hipError_t launch2(const GemvPart* parts, int count, int nb, const uint16_t* x, int batch,
                   int64_t ldx, const Force& f, hipStream_t s) {
  switch (batch) {
    case 1: return launch3<LAYOUT, XT, 1, NP>(parts, count, nb, x, ldx, f, s);
    case 2: return launch3<LAYOUT, XT, 2, NP>(parts, count, nb, x, ldx, f, s);
    case 3: return launch3<LAYOUT, XT, 3, NP>(parts, count, nb, x, ldx, f, s);
    case 4: return launch3<LAYOUT, XT, 4, NP>(parts, count, nb, x, ldx, f, s);
    case 5: return launch3<LAYOUT, XT, 5, NP>(parts, count, nb, x, ldx, f, s);
    case 6: return launch3<LAYOUT, XT, 6, NP>(parts, count, nb, x, ldx, f, s);
    case 7: return launch3<LAYOUT, XT, 7, NP>(parts, count, nb, x, ldx, f, s);
    default: return launch3<LAYOUT, XT, 8, NP>(parts, count, nb, x, ldx, f, s);
  }
}

// Entry for one activation dtype (each dtype is compiled in its own translation unit).
template <int XT>
hipError_t launch_gemv_xt(const GemvPart* parts, int count, int layout, int nb, const uint16_t* x,
                          int batch, int64_t ldx, const Force& f, hipStream_t s) {
  if (count == 1)
    return layout == kDual ? launch2<kDual, XT, 1>(parts, count, nb, x, batch, ldx, f, s)
                           : launch2<kFast, XT, 1>(parts, count, nb, x, batch, ldx, f, s);
  return layout == kDual ? launch2<kDual, XT, kMaxGemvParts>(parts, count, nb, x, batch, ldx, f, s)
                         : launch2<kFast, XT, kMaxGemvParts>(parts, count, nb, x, batch, ldx, f, s);
}

}  // namespace
}  // namespace rfp4
