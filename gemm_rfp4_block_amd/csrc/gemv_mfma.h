// GEMV on the matrix cores ("Feasibility Report: Porting ROCmFP4 to Atlas", "Kernel
// System": the decode gemv), for activation batches of 1..8 rows.
//
//   y[b][r] = sum_c weight(r, c) * x[b][c]
//
// Mapping. A workgroup of four wavefronts (one per SIMD) owns 16 consecutive weight
// rows (one MFMA tile of v_mfma_f32_16x16x32_{f16,bf16}), or R = 2 such tiles (32 rows,
// two accumulators per wavefront sharing each activation fragment) for batches above 4
// on large launches. Lane l of a wavefront serves
// as B-operand lane for weight row l % 16 and as A-operand lane for activation row
// l % 16 (rows beyond the batch read a clamped, finite row whose results are never
// stored); the lane group g = 4 w + l / 16 (w the wavefront) multiplies units g, g + 16,
// g + 32, ... of the row (a unit is P = 1 or 2 consecutive blocks). The weights are
// loaded along rows and handed to these lanes through an LDS stage per chunk (below).
// The sum over k is order free, so each MFMA adds, for every lane group, 8 consecutive
// weights of that lane's own unit against the matching 8 activations: block j gives four MFMA steps s = 0..3 over weights 8s .. 8s+7 (low
// nibbles of qs words 0, 1 / 2, 3, then the high nibbles), and the activations of step
// s are the 16-byte piece s of the block.
//
// Activations. The 16 lane groups consume the units of a row in chunks of 16 (chunk
// t = units 16t .. 16t + 15). Each chunk's activations, for all batch rows, are staged
// in LDS just before it is multiplied, and so are its weights (each lane stores the
// unit it loaded and reads back the unit it multiplies); the loads are issued two
// chunks ahead into registers, activations and weights of a chunk together, so that
// the staging waits only for loads that are due anyway. Per chunk the workgroup reads
// batch x 16 units of activations from the L2; staging the whole activation matrix up
// front, or having every lane read its activations from global memory, measured 1.2 to
// 1.6 times slower. Four wavefronts per workgroup measured faster than 8 or 16 on every
// decode shape (smaller barriers, more registers per wavefront) and faster than 2.
//
// Decode. Each workgroup builds a 128-entry LDS table: for every value of a scale byte's
// low seven bits, the f16 (or bf16) encodings of the eight magnitudes times the decoded
// scale, as a plane of low bytes and a plane of high bytes. Every such product is exact
// in both formats (at most 8 significant bits, between 2^-10 and 2400). Four weights
// then take two v_perm_b32 gathers, an OR of the sign bits into the high bytes and two
// interleaving v_perm_b32; the scale is part of the table, so the MFMA products are the
// exact weight times activation products, summed in fp32.
//
// The four wavefronts' 16 x 16 accumulator tiles are added in LDS in a fixed order and
// the batch rows are stored. Long rows on few tiles split each tile's chunks between
// two to four workgroups (see mfma_splits); the last of them to finish adds the parts in
// a fixed order.

#pragma once

#include <type_traits>

#include "gemv_impl.h"

namespace rfp4 {
namespace {

typedef _Float16 mf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mbf16x8 __attribute__((ext_vector_type(8)));
typedef float mf32x4 __attribute__((ext_vector_type(4)));

template <int XT>
struct MfmaOps;

template <>
struct MfmaOps<kF16> {
  static __device__ __forceinline__ mf32x4 mfma(uint4 a, uint4 b, mf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf16x8, a),
                                                  __builtin_bit_cast(mf16x8, b), c, 0, 0, 0);
  }
  // Encoding of an exactly representable value.
  static __device__ __forceinline__ uint32_t enc(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
};

template <>
struct MfmaOps<kBF16> {
  static __device__ __forceinline__ mf32x4 mfma(uint4 a, uint4 b, mf32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mbf16x8, a),
                                                   __builtin_bit_cast(mbf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t enc(float v) { return __float_as_uint(v) >> 16; }
};

// Four weights of one nibble plane: `idx` holds their 3-bit magnitude indices in bytes
// 0..3, `sgn` their sign bits at bit 7 of bytes 0..3, `t` the table entry of the scale
// (low-byte plane of magnitudes 0-3, 4-7, then the high-byte plane). Returns the 16-bit
// encodings of weights 0, 1 and 2, 3 as two words.
__device__ __forceinline__ uint2 decode_plane(uint32_t idx, uint32_t sgn, uint4 t) {
  const uint32_t lo = __builtin_amdgcn_perm(t.y, t.x, idx);
  const uint32_t hi = __builtin_amdgcn_perm(t.w, t.z, idx) | sgn;
  return uint2{__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u)};
}

// The two scale bytes of block B of a unit (dual: e0, e1; fast: e, e).
template <int LAYOUT, int P, int B>
__device__ __forceinline__ void unit_scale_bytes(const UnitRaw<P>& u, uint32_t& e0, uint32_t& e1) {
  constexpr int off = (P == 1) ? 16 : B * block_bytes(LAYOUT) + 16;
  constexpr int wi = off / 4;
  constexpr int bi = off % 4;
  const uint32_t word = u.d[wi] >> (8 * bi);
  e0 = word & 0x7Fu;
  e1 = LAYOUT == kDual ? (word >> 8) & 0x7Fu : e0;
}

constexpr int kMfmaWaves = 4;

// Polls of the arrival counter by a combining part before it falls back to storing and
// counting its own sums (each poll is a round trip to the coherence point plus a short
// sleep: together a few microseconds, longer than the parts normally lag each other).
constexpr int kCombinerPolls = 24;

template <int LAYOUT, int XT, int P, bool BIG, int R, int NP>
__global__ __launch_bounds__(64 * kMfmaWaves) void gemv_mfma_kernel(const GemvParts<NP> parts, int nu,
                                                           const uint16_t* __restrict__ x,
                                                           int64_t ldx, int batch, int splits,
                                                           float* __restrict__ partial,
                                                           int* __restrict__ arrivals, int polls) {
  constexpr int W = kMfmaWaves;
  constexpr int UB = P * block_bytes(LAYOUT);
  constexpr int THREADS = 64 * W;
  constexpr int G = 4 * W;        // lane groups: units of a row per chunk
  constexpr int PU = 4 * P;       // 16-byte activation pieces per unit
  constexpr int XPT = BIG ? 2 * P : P;  // pieces per thread per chunk: batch <= 8 or <= 4
  // Chunks in flight. Two rather than three: 113-116 instead of 140-146 registers at
  // batches above 4 (one tile per workgroup), so four workgroups fit on a CU instead of
  // three, which the k-range split below turns into more wavefronts per CU; measured
  // (same box, us) 5120 x 17408 batch 3/8 19.0/23.5 -> 17.8/22.2 at the same split,
  // 5120 x 6144 batch 8 12.0 -> 11.2, 17408 x 5120 batch 4 16.7 -> 16.0.
  constexpr int D = 2;
  // LDS pieces per activation row of a chunk: G units of PU + 1 pieces, plus one piece so
  // that consecutive rows start 16 bytes apart modulo 256. The 16 lanes of a lane group
  // read the same piece of up to 8 different rows in one access; with rows a multiple of
  // 256 bytes apart those reads would all fall on the same four banks.
  constexpr int XROW = G * (PU + 1) + 1;
  typedef MfmaOps<XT> M;
  extern __shared__ uint4 smem_m[];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;  // weight row of the tile (B) and activation row (A)
  const int g = 4 * wv + (lane >> 4);  // lane group: unit g of each chunk
  uint4* const lut = smem_m;
  uint4* const xs = smem_m + 128;  // chunk: batch rows of XROW pieces
  mf32x4* const red = reinterpret_cast<mf32x4*>(xs);  // reused after the last chunk
  // Weight stage of a chunk, after its activations: the (realigned) words of unit u of
  // tile row r in planes of 16-byte slots (words 0-3, and 4-7 for pairs) and 4-byte slots
  // (the last word), slot q * 256 + u * 16 + (r ^ u) for tile q. The 16 lanes that store
  // one row's units and the 16 lanes that read one unit of every row both touch 16
  // distinct slot positions modulo 16, i.e. distinct banks.
  uint4* const ws_a = xs + batch * XROW;
  uint4* const ws_b = ws_a + R * 256;  // pairs only
  uint32_t* const ws_c = reinterpret_cast<uint32_t*>(ws_a + R * 256 * (P == 2 ? 2 : 1));

  // Tile and part of this workgroup: the grid is tiles x splits, part p of a tile taking
  // its chunks [p T_all / splits, (p + 1) T_all / splits) (the plan keeps splits <= T_all).
  const int tiles = static_cast<int>(gridDim.x) / splits;
  const int tile = static_cast<int>(blockIdx.x) % tiles;
  const int part = static_cast<int>(blockIdx.x) / tiles;
  int mi = 0;
  if constexpr (NP > 1)
    while (mi + 1 < parts.count && tile >= parts.gbeg[mi + 1]) ++mi;
  const int n_part = NP > 1 ? parts.n[mi] : parts.n[0];
  const int r0 = (tile - (NP > 1 ? parts.gbeg[mi] : 0)) * 16 * R;
  const int64_t rowbytes = static_cast<int64_t>(nu) * UB;
  // Weight loads run along rows: lane l of wavefront w loads unit l % 16 of the chunk
  // from tile row 4 w + l / 16, so each load instruction reads 16 consecutive units of
  // four rows (the MFMA lane of a (row, unit) pair holds one unit of each of 16 rows,
  // which would make every instruction touch 16 rows). The units reach their MFMA lanes
  // through the weight stage in LDS.
  static_assert(W == 4, "the weight stage maps 4 wavefronts x 4 lane groups to 16 rows and 16 units");
  const int lrow = 4 * wv + (lane >> 4);
  const int lunit = lane & 15;
  const uint8_t* wrow[R];
#pragma unroll
  for (int q = 0; q < R; ++q)
    wrow[q] = (NP > 1 ? parts.w[mi] : parts.w[0]) + static_cast<int64_t>(min(r0 + 16 * q + lrow, n_part - 1)) * rowbytes;

  // Chunk c covers units G c .. G c + G - 1 of every row: lane group g multiplies unit
  // G c + g (past the row end the address is clamped). This part's chunks are
  // c = t_off + t, t < T.
  const int T_all = (nu + G - 1) / G;
  const int t_off = part * T_all / splits;
  const int T = (part + 1) * T_all / splits - t_off;
  auto unit_ptr = [&](int q, int t) { return wrow[q] + static_cast<int64_t>(min(G * (t_off + t) + lunit, nu - 1)) * UB; };

  // Activation chunk t: piece i = (b G + u) PU + p is the 16-byte piece p of unit G t + u
  // of activation row b, stored at LDS unit b XROW + u (PU + 1) + p; consecutive threads
  // read consecutive pieces of a row. The loads are clamped to the last piece (and to
  // the row's last unit), so every thread loads XPT pieces in bounds; pieces of units
  // past the row end are stored as zeros, so the weights there meet zeros (0 * inf would
  // be NaN). The zeroing happens at the LDS store, which waits for the load anyway: a
  // select applied to the loaded registers is free to be placed anywhere after the load,
  // and placed early it makes the wavefront wait for loads of chunks still meant to be in
  // flight.
  const int pieces = batch * G * PU;
  struct XChunk {
    uint4 v[XPT];
  };
  auto x_load = [&](int t) {
    XChunk c;
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = min(static_cast<int>(threadIdx.x) + j * THREADS, pieces - 1);
      const int p = i % PU;
      const int bu = i / PU;
      const int b = bu / G;
      const int unit = G * (t_off + t) + (bu % G);
      c.v[j] = *reinterpret_cast<const uint4*>(x + b * ldx + 32 * P * min(unit, nu - 1) + 8 * p);
    }
    return c;
  };
  // Only a chunk that reaches past the row end holds dead pieces (a uniform test), so
  // the others store the loaded registers as they are; the piece count is a multiple of
  // the block size for the first pieces / THREADS stores of every thread (uniform too).
  auto x_store = [&](const XChunk& c, int t) {
    const bool ragged = G * (t_off + t + 1) > nu;
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = static_cast<int>(threadIdx.x) + j * THREADS;
      if ((j + 1) * THREADS <= pieces || i < pieces) {
        const int bu = i / PU;
        uint4 v = c.v[j];
        if (ragged) {
          const uint32_t m = G * (t_off + t) + (bu % G) < nu ? ~0u : 0u;
          v = uint4{v.x & m, v.y & m, v.z & m, v.w & m};
        }
        xs[(bu / G) * XROW + (bu % G) * (PU + 1) + i % PU] = v;
      }
    }
  };

  // D chunks in flight: the activations and weights of chunk t are loaded together,
  // so the LDS stores of chunk t wait for exactly those loads and leave the later chunks
  // in flight.
  XChunk xr[D];
  UnitRaw<P> rb[R][D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int tc = min(d, T - 1);  // straight-line loads; a chunk past T is never used
    xr[d] = x_load(tc);
#pragma unroll
    for (int q = 0; q < R; ++q) load_unit<LAYOUT, P>(unit_ptr(q, tc), rb[q][d]);
  }

  // Decode table (threads 0..127), built while the first chunks' loads are in flight
  // (before them it delayed every workgroup's first request: 1-3 % on most launches).
  if (threadIdx.x < 128) {
    const float sv = scale_exact(threadIdx.x);
    const float mags[8] = {0.f, 1.f, 2.f, 3.f, 4.f, 6.f, 8.f, 10.f};
    uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t e = M::enc(mags[i] * sv);
      lo[i >> 2] |= (e & 0xFFu) << (8 * (i & 3));
      hi[i >> 2] |= (e >> 8) << (8 * (i & 3));
    }
    lut[threadIdx.x] = uint4{lo[0], lo[1], hi[0], hi[1]};
  }

  auto w_store = [&](int d) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const UnitRaw<P> ua = unit_aligned<LAYOUT, P>(rb[q][d]);
      const int sl = q * 256 + lunit * 16 + (lrow ^ lunit);
      ws_a[sl] = uint4{ua.d[0], ua.d[1], ua.d[2], ua.d[3]};
      if constexpr (P == 2) {
        ws_b[sl] = uint4{ua.d[4], ua.d[5], ua.d[6], ua.d[7]};
        ws_c[sl] = ua.d[8];
      } else {
        ws_c[sl] = ua.d[4];
      }
    }
  };
  // The unit this lane multiplies (tile row col, unit g of the chunk), from the stage.
  auto w_read = [&](int q) {
    const int sl = q * 256 + g * 16 + (col ^ g);
    UnitRaw<P> u;
    const uint4 a = ws_a[sl];
    u.d[0] = a.x;
    u.d[1] = a.y;
    u.d[2] = a.z;
    u.d[3] = a.w;
    if constexpr (P == 2) {
      const uint4 b = ws_b[sl];
      u.d[4] = b.x;
      u.d[5] = b.y;
      u.d[6] = b.z;
      u.d[7] = b.w;
      u.d[8] = ws_c[sl];
    } else {
      u.d[4] = ws_c[sl];
    }
    u.sh = 0;
    return u;
  };


  const int xb = min(col, batch - 1);  // activation row of this A lane (clamped)
  mf32x4 acc[R];
#pragma unroll
  for (int q = 0; q < R; ++q) acc[q] = mf32x4{0.f, 0.f, 0.f, 0.f};

  // A lane group past the row end holds the row's last unit of weights against zeroed
  // activations, so it adds zeros.
  auto consume = [&](int d) {
    (void)d;  // the chunk's weights are in the stage, its activations in xs
    const uint4* const xu = xs + xb * XROW + g * (PU + 1);
    UnitRaw<P> ua[R];
#pragma unroll
    for (int q = 0; q < R; ++q) ua[q] = w_read(q);
    auto block = [&](auto b_c) {
      constexpr int B = decltype(b_c)::value;
      uint4 q4[R], t0[R], t1[R];
#pragma unroll
      for (int q = 0; q < R; ++q) {
        q4[q] = unit_qs<LAYOUT, P, B>(ua[q]);
        uint32_t e0, e1;
        unit_scale_bytes<LAYOUT, P, B>(ua[q], e0, e1);
        t0[q] = lut[e0];
        t1[q] = LAYOUT == kDual ? lut[e1] : t0[q];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 a = xu[4 * B + s];
#pragma unroll
        for (int q = 0; q < R; ++q) {
          const uint32_t qw[4] = {q4[q].x, q4[q].y, q4[q].z, q4[q].w};
          const uint32_t qa = qw[2 * (s & 1)], qb = qw[2 * (s & 1) + 1];
          uint2 pa, pb;
          if (s < 2) {  // low nibbles: first half (scale e0)
            pa = decode_plane(qa & 0x07070707u, (qa << 4) & 0x80808080u, t0[q]);
            pb = decode_plane(qb & 0x07070707u, (qb << 4) & 0x80808080u, t0[q]);
          } else {  // high nibbles: second half (scale e1)
            pa = decode_plane((qa >> 4) & 0x07070707u, qa & 0x80808080u, t1[q]);
            pb = decode_plane((qb >> 4) & 0x07070707u, qb & 0x80808080u, t1[q]);
          }
          acc[q] = M::mfma(a, uint4{pa.x, pa.y, pb.x, pb.y}, acc[q]);
        }
      }
    };
    block(std::integral_constant<int, 0>{});
    if constexpr (P == 2) block(std::integral_constant<int, 1>{});
  };

  // Per chunk: wait until every wavefront is done with the previous chunk, store this
  // one, wait until it is complete, multiply; then issue chunk t + D. Rounds of D
  // chunks keep the register rings indexed by constants. Every round but the last
  // loads unconditionally (clamped to the last chunk), since a path that skipped loads
  // would make the compiler's load waits count the shortest path; the last round loads
  // nothing and skips the chunks past T, so no load outlives the last multiply. The
  // first barrier also orders the table writes before their first reads.
  int t = 0;
  for (; t + D < T; t += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (t + d > 0) __syncthreads();
      x_store(xr[d], t + d);
      w_store(d);
      __syncthreads();
      consume(d);
      const int tn = min(t + d + D, T - 1);
      xr[d] = x_load(tn);
#pragma unroll
      for (int q = 0; q < R; ++q) load_unit<LAYOUT, P>(unit_ptr(q, tn), rb[q][d]);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (t + d < T) {
      if (t + d > 0) __syncthreads();
      x_store(xr[d], t + d);
      w_store(d);
      __syncthreads();
      consume(d);
    }
  }

  // Lane l, register i holds batch row 4 (l / 16) + i of weight row l % 16.
  float* const y = NP > 1 ? parts.y[mi] : parts.y[0];
  const int64_t ldy = NP > 1 ? parts.ldy[mi] : parts.ldy[0];
  __syncthreads();  // the last chunk's reads are done before its LDS is reused
#pragma unroll
  for (int q = 0; q < R; ++q) red[(q * W + wv) * 64 + lane] = acc[q];
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int q = 0; q < R; ++q) {
    for (int w = 1; w < W; ++w) {
      const mf32x4 o = red[(q * W + w) * 64 + lane];
      acc[q][0] += o[0];
      acc[q][1] += o[1];
      acc[q][2] += o[2];
      acc[q][3] += o[3];
    }
  }
  const int row = r0 + col;
  if (R == 1 && splits > 1) {
    // Parts leave their sums (tile-major, weight row, batch row) and count themselves;
    // one part adds all parts in part order, so the result does not depend on the
    // arrival order.
    // Ordering. Every access to the sums and counters is an agent-scope atomic, which
    // gfx950 code carries out at the device's coherence point: the stores write
    // through (sc1), the loads bypass the non-coherent caches (sc1), the counter is an
    // atomic read-modify-write. s_waitcnt(0) holds the counter update back until every
    // store of this wavefront has completed, so a part that counts itself has its sums
    // in coherent memory; the combining part's loads are issued only after its counter
    // update, or its poll of the counter, has returned the value that lets them run, so
    // they read every counted part's sums. A release on the counter and an acquire after
    // it would compile to the same instructions plus a write-back and an invalidation of
    // the whole L2 (buffer_wbl2 sc1, buffer_inv sc1), which only matter for data written
    // or read without sc1 (there is none here) and measured 3-5x slower on these launches.
    // Combining. The last part (dispatched last, so normally the last to finish) is the
    // combiner: it polls the arrival counter (a bounded number of times) until the other
    // splits - 1 parts have counted themselves, then reads their sums and adds its own
    // from registers, without storing them or counting itself; that saves the round trips
    // of its own stores and counter update at the end of the launch. A combiner that
    // stops polling before the others have arrived falls back to the general protocol:
    // it stores and counts itself like the others, and whichever part counts last adds
    // all parts from memory. Either way the parts are added in part order, so the result
    // does not depend on which path ran, and the poll is bounded, so no wavefront waits
    // for another indefinitely. The counter is reset by the part that combined (every
    // other part has counted itself by then).
    const bool combiner = part == splits - 1;
    int seen = 0;
    if (combiner && lane == 0) {
      for (int it = 0; it < polls; ++it) {
        seen = __hip_atomic_load(&arrivals[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen == splits - 1) break;
        __builtin_amdgcn_s_sleep(4);
      }
    }
    const bool fast = combiner && __shfl(seen, 0, 64) == splits - 1;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (!fast) {
      float* const mine = partial + (static_cast<int64_t>(part) * tiles + tile) * 128;
      if (lane < 32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(&mine[col * 8 + 4 * (lane >> 4) + i], acc[0][i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      int prior = 0;
      if (lane == 0) prior = __hip_atomic_fetch_add(&arrivals[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__shfl(prior, 0, 64) != splits - 1) return;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    if (lane < 32 && row < n_part) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * (lane >> 4) + i;
        if (b < batch) {
          float sum = 0.f;
          for (int q = 0; q < splits; ++q)
            sum += (fast && q == splits - 1)
                       ? acc[0][i]
                       : __hip_atomic_load(&partial[(static_cast<int64_t>(q) * tiles + tile) * 128 + col * 8 + b],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          y[b * ldy + row] = sum;
        }
      }
    }
    if (lane == 0) __hip_atomic_store(&arrivals[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    if (row + 16 * q < n_part) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = 4 * (lane >> 4) + i;
        if (b < batch) y[b * ldy + row + 16 * q] = acc[q][i];
      }
    }
  }
}

struct MfmaPlan {
  int p, nu, tiles, splits, r;
  bool big;
  size_t shm;
};

// Split chunks: launches of long rows and few tiles give each tile's chunks to several
// workgroups, so that every CU gets more wavefronts. Measured over 1024-12288 rows of
// 17408 columns and rows of 6144-13824 columns (graph-replayed launches, batches 3-8), a
// launch takes about a fixed time plus a per-chunk cost times the chunks that the
// busiest CU's workgroups hold together, ceil(tiles s / CUs) ceil(chunks / s), with a
// ~15 % higher per-chunk cost where every CU holds at most one workgroup (one
// workgroup's wavefronts leave the loads less overlapped). The launcher takes the split
// s (1 to kMaxSplits) of the lowest such cost, the smaller s on a tie, among those whose
// workgroups all fit on the CUs at once (`slots`: resident workgroups per CU, from the
// occupancy of the kernel instance, times the CUs) and whose parts keep at least
// kMinSplitChunks chunks each (shorter parts lose what they gain to the combining
// step). Measured (same box, us, parts 1/2/3/4, * = chosen): 5120 x 17408 batch 8
// 23.6/22.4/21.3*/22.1, 4096 x 17408 batch 8 18.1/17.1*/18.1/18.5, 8192 x 17408 batch 8
// 25.0*/27.9/29.0/30.0, 1024 x 17408 batch 8 17.7/13.3/11.4*/11.2 (four parts leave four
// chunks), 4096 x 8192 batch 8 10.3*/11.2/11.9/12.0, 5120 x 6144 batch 8 11.1*/12.2/11.5/13.5.
// The partial sums and arrival counters live in a per-(device, stream) workspace of fixed
// size: the counters first (a region for up to kMaxSplitTiles tiles, zero at allocation
// and reset by the last arrival of each tile), then the sums of up to kMaxSplits parts.
// A forced split (rfp4_force, 1-4 parts) is reduced to at least one chunk per part.
constexpr int kMaxSplitTiles = 1024;
constexpr int kMaxSplits = 4;
constexpr int kMinSplitChunks = 5;
constexpr size_t kSplitCounterBytes = kMaxSplitTiles * sizeof(int);
constexpr size_t kSplitWorkspaceBytes =
    kSplitCounterBytes + static_cast<size_t>(kMaxSplits) * kMaxSplitTiles * 128 * sizeof(float);
inline int mfma_splits(int tiles, int nu, int64_t slots, const Force& force) {
  const int t_all = (nu + 4 * kMfmaWaves - 1) / (4 * kMfmaWaves);
  const int64_t cus = device_cu_count();
  int s = 1;
  int64_t best = 0;
  for (int c = 1; c <= kMaxSplits; ++c) {
    const int64_t wgs = static_cast<int64_t>(tiles) * c;
    if (c > 1 && (wgs > slots || t_all / c < kMinSplitChunks)) continue;
    // 20 x the cost above: the lone-workgroup factor 1.15 as 23 / 20.
    const int64_t cost = (wgs + cus - 1) / cus * ((t_all + c - 1) / c) * (wgs <= cus ? 23 : 20);
    if (c == 1 || cost < best) {
      best = cost;
      s = c;
    }
  }
  if (force.gemv_splits != 0) s = force.gemv_splits;
  if (tiles > kMaxSplitTiles) s = 1;
  if (s > t_all) s = t_all;
  return s;
}

// LDS of a launch: the table plus one activation chunk and its weight stage (or the
// cross-wavefront sums, if larger).
inline size_t mfma_lds(int p, int batch, int r) {
  const size_t chunk = static_cast<size_t>(batch) * (4 * kMfmaWaves * (4 * p + 1) + 1) * 16 +
                       static_cast<size_t>(r) * 256 * (p == 2 ? 36 : 20);
  const size_t red = static_cast<size_t>(r) * kMfmaWaves * 64 * 16;
  return 128 * 16 + (chunk > red ? chunk : red);
}

inline MfmaPlan mfma_plan(const GemvPart* parts, int count, int nb, int batch, const Force& force) {
  MfmaPlan pl;
  pl.p = nb % 2 == 0 ? 2 : 1;
  pl.nu = nb / pl.p;
  int tiles16 = 0;
  for (int i = 0; i < count; ++i) tiles16 += static_cast<int>((parts[i].n + 15) / 16);
  pl.big = batch > 4;
  // Two tiles per workgroup (sharing each staged activation chunk) for batches above 4
  // on launches of at least six 16-row tiles per CU. Measured against one tile per
  // workgroup (same box, us, batch 5 / batch 8): 152064 x 5120 104.2 / 111.9 against
  // 115.5 / 127.6, 32768 x 5120 26.3 / 27.8 against 27.8 / 30.7, 24576 x 5120 20.5 / 21.7
  // against 21.5 / 24.1, fused gate + up (2 x 17408 rows) 29.6 / 31.6 against 29.9 / 33.0;
  // below six tiles per CU one tile per workgroup (four workgroups per CU) is ahead:
  // 20480 x 5120 19.8 / 21.0 against 18.9 / 21.3, 17408 x 5120 19.5 / 20.6 against
  // 17.4 / 19.6. At batches <= 4 two tiles were slower (17408 x 5120 batch 2 16.7 -> 19.4).
  pl.r = (pl.big && tiles16 >= 6 * device_cu_count()) ? 2 : 1;
  pl.tiles = 0;
  for (int i = 0; i < count; ++i) pl.tiles += static_cast<int>((parts[i].n + 16 * pl.r - 1) / (16 * pl.r));
  pl.shm = mfma_lds(pl.p, batch, pl.r);
  pl.splits = 1;  // set by the launcher (it depends on the kernel instance's occupancy)
  return pl;
}

// Workgroups of a one-tile kernel instance that fit on a CU at once (its registers and
// the LDS of its largest batch), from the runtime's occupancy calculator; computed once
// per instance.
template <int LAYOUT, int XT, int P, bool BIG, int NP>
int mfma_resident() {
  static const int n = [] {
    int b = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b, reinterpret_cast<const void*>(&gemv_mfma_kernel<LAYOUT, XT, P, BIG, 1, NP>), 64 * kMfmaWaves,
        mfma_lds(P, BIG ? 8 : 4, 1));
    return e == hipSuccess && b > 0 ? b : 1;
  }();
  return n;
}

template <int LAYOUT, int XT, int P, bool BIG, int NP>
hipError_t launch_mfma_p(const MfmaPlan& pl, const GemvParts<NP>& gp, const uint16_t* x, int64_t ldx,
                         int batch, float* partial, int* arrivals, int polls, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(pl.tiles) * pl.splits), block(64 * kMfmaWaves);
  if (BIG && pl.r == 2)
    gemv_mfma_kernel<LAYOUT, XT, P, BIG, BIG ? 2 : 1, NP><<<grid, block, pl.shm, stream>>>(
        gp, pl.nu, x, ldx, batch, pl.splits, partial, arrivals, polls);
  else
    gemv_mfma_kernel<LAYOUT, XT, P, BIG, 1, NP><<<grid, block, pl.shm, stream>>>(
        gp, pl.nu, x, ldx, batch, pl.splits, partial, arrivals, polls);
  return hipGetLastError();
}

template <int LAYOUT, int XT, int NP>
hipError_t launch_mfma(const GemvPart* parts, int count, int nb, const uint16_t* x, int batch,
                       int64_t ldx, const Force& force, hipStream_t stream) {
  MfmaPlan pl = mfma_plan(parts, count, nb, batch, force);
  if (pl.r == 1) {
    const int resident = pl.p == 2 ? (pl.big ? mfma_resident<LAYOUT, XT, 2, true, NP>()
                                             : mfma_resident<LAYOUT, XT, 2, false, NP>())
                                   : (pl.big ? mfma_resident<LAYOUT, XT, 1, true, NP>()
                                             : mfma_resident<LAYOUT, XT, 1, false, NP>());
    pl.splits = mfma_splits(pl.tiles, pl.nu, static_cast<int64_t>(resident) * device_cu_count(), force);
  }
  float* partial = nullptr;
  int* arrivals = nullptr;
  if (pl.splits > 1) {
    // Always the fixed maximum, so the workspace is allocated once and never replaced.
    void* ws = nullptr;
    if (stream_workspace(kWorkspaceGemv, stream, kSplitWorkspaceBytes, true, &ws) != hipSuccess) {
      pl.splits = 1;  // no workspace (first call under graph capture, or no memory): no split
    } else {
      arrivals = static_cast<int*>(ws);
      partial = reinterpret_cast<float*>(static_cast<char*>(ws) + kSplitCounterBytes);
    }
  }
  const int polls = force.gemv_split_combine == 1 ? 0 : kCombinerPolls;
  GemvParts<NP> gp;
  gp.count = count;
  gp.gbeg[0] = 0;
  for (int i = 0; i < count; ++i) {
    gp.w[i] = parts[i].w;
    gp.y[i] = parts[i].y;
    gp.ldy[i] = parts[i].ldy;
    gp.n[i] = static_cast<int>(parts[i].n);
    gp.gbeg[i + 1] = gp.gbeg[i] + static_cast<int>((parts[i].n + 16 * pl.r - 1) / (16 * pl.r));
  }
  if (pl.p == 2)
    return pl.big ? launch_mfma_p<LAYOUT, XT, 2, true, NP>(pl, gp, x, ldx, batch, partial, arrivals, polls, stream)
                  : launch_mfma_p<LAYOUT, XT, 2, false, NP>(pl, gp, x, ldx, batch, partial, arrivals, polls, stream);
  return pl.big ? launch_mfma_p<LAYOUT, XT, 1, true, NP>(pl, gp, x, ldx, batch, partial, arrivals, polls, stream)
                : launch_mfma_p<LAYOUT, XT, 1, false, NP>(pl, gp, x, ldx, batch, partial, arrivals, polls, stream);
}

// Matrix-core path for the launches where it is faster. Measured (graph-replayed
// launches over rotating weight copies, one machine, dot-product / matrix cores, us):
// the dot-product kernel wins at batch 1 (its decode needs no table, no staging and no
// cross-wave reduction). At batch 2 the matrix cores win from 4096 to 65536 rows (all
// matrices of the launch together): 4096 x 5120 7.52 / 6.68, 8192 x 5120 9.00 / 8.64,
// 17408 x 5120 15.56 / 14.73, 4096 x 17408 14.52 / 14.11, 5120 x 17408 17.48 / 16.70,
// 5120 x 6144 9.45 / 8.99, fused q + k + v (7168 rows) 11.11 / 8.62, even at 12288 (11.21 /
// 11.29), 49152 (33.05 / 32.76) and 69632 rows (45.02 / 44.87); the dot-product kernel
// below (1024 x 5120 4.77 / 6.06, 2048 x 5120 5.92 / 6.25, 2048 x 17408 10.00 / 11.00,
// 3072 x 17408 12.42 / 13.74; 3072 x 5120 7.21 / 6.51 is the exception) and above
// (152064 x 5120 93.6 / 95.9). From batch 3 the matrix cores win (their decode does not
// grow with the batch), except on one matrix of at most 1024 short rows up to batch 6
// (1024 x 5120 batch 3/4/6 5.68 / 6.26, 6.25 / 6.46, 7.26 / 7.15; at batch 8 8.75 / 7.66,
// and from 2048 rows the tiles lead). A forced kernel (rfp4_force) replaces the choice.
inline bool use_mfma(const GemvPart* parts, int count, int nb, int batch, const Force& force) {
  if (force.gemv_kernel == RFP4_GEMV_KERNEL_DOT) return false;
  if (force.gemv_kernel == RFP4_GEMV_KERNEL_TILES) return true;
  if (batch < 2) return false;
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) rows += parts[i].n;
  if (batch == 2) return rows >= 4096 && rows <= 65536;
  if (batch <= 6 && count == 1 && rows <= 1024 && nb <= 192) return false;
  return true;
}

template <int XT>
hipError_t launch_gemv_mfma_xt(const GemvPart* parts, int count, int layout, int nb, const uint16_t* x,
                               int batch, int64_t ldx, const Force& f, hipStream_t s) {
  if (count == 1)
    return layout == kDual ? launch_mfma<kDual, XT, 1>(parts, count, nb, x, batch, ldx, f, s)
                           : launch_mfma<kFast, XT, 1>(parts, count, nb, x, batch, ldx, f, s);
  return layout == kDual ? launch_mfma<kDual, XT, kMaxGemvParts>(parts, count, nb, x, batch, ldx, f, s)
                         : launch_mfma<kFast, XT, kMaxGemvParts>(parts, count, nb, x, batch, ldx, f, s);
}

}  // namespace
}  // namespace rfp4
