// Weight-only 4-bit GEMM for prefill: C[m][r] = bf16( sum_c A[m][c] * W[r][c] ).
//
// The page names this kernel w4a16_gemm, a weight-only 4-bit GEMM for prefill
// ("Feasibility Report: Porting ROCmFP4 to Atlas", "Kernel System"). Prefill is a
// dense contraction, so it runs on the matrix cores: each workgroup decodes a tile of
// packed weights into LDS as bf16 (exact: every codebook value times every decoded
// scale is a bf16 value) and feeds v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
// the epilogue rounds to bf16 (nearest even).
//
// Tiling. A 512-thread workgroup (8 wavefronts, two per SIMD) owns a 256 x 256 tile of
// C (256 rows of A by 256 weight rows). Each step consumes 64 columns of K, i.e. two
// ROCmFP4 blocks per weight row; each wavefront computes a 64 x 128 sub-tile as 2 x 4
// MFMA tiles of 32 x 32, 128 fp32 accumulators per lane.
//
// Pipeline (LDS double-buffered, one barrier per step). While step s is multiplied out
// of LDS buffer s % 2:
//   * the A tile of step s+1 is loaded into registers (four 16-byte chunks per thread)
//     and written to the other buffer after the MFMAs;
//   * the packed weights of step s+1 (loaded one step earlier, one block per thread)
//     are decoded to bf16 into the other buffer, one 16-byte chunk per 16-column k slice,
//     interleaved with that slice's MFMAs; the weights of step s+2 are loaded.
// LDS rows are 64 bf16 (eight 16-byte chunks) with the chunk index XOR-swizzled by the
// row, so the MFMA fragment reads (32 consecutive rows, one chunk) hit distinct banks.
//
// Mapping. Workgroups are dispatched round-robin over the 8 XCDs; with the M-tile index
// taken as (workgroup id mod M-tiles), all workgroups of an XCD share the same 256 rows
// of A (2.6 MB at K = 5120), which stay in that XCD's L2.

#include "rfp4_decode.h"
#include "rfp4_internal.h"

namespace rfp4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int kTileBytes = BM * BK * 2;  // one bf16 tile of A or W in LDS (32 KB)

// Byte offset of 16-byte chunk c (0..7) of row r in a swizzled LDS tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  // Both values are exactly representable in bf16, so the conversion is exact.
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// Decode chunk c (weights 8c .. 8c+7) of one block to bf16 (c * S, exact) and write it
// to chunk c0 + c of LDS row r. Chunks 0, 1 are the low nibbles of qs words 2c, 2c+1
// (first half, scale e0); chunks 2, 3 the high nibbles of qs words 2(c-2), 2(c-2)+1
// (second half, scale e1; the fast layout has one scale).
template <int LAYOUT, int C>
__device__ __forceinline__ void decode_chunk_to_lds(const BlockRaw& b, char* tile, int r, int c0) {
  const float s = scale_exact((C < 2 || LAYOUT == kFast) ? (b.sc & 0xFFu) : (b.sc >> 8));
  const uint32_t q[4] = {b.qs.x, b.qs.y, b.qs.z, b.qs.w};
  uint32_t o[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t word = q[2 * (C & 1) + h];
    const uint32_t codes = (C < 2) ? codes_low(word) : codes_high(word);
    const f32x2 lo = pair_f32(codes, false);
    const f32x2 hi = pair_f32(codes, true);
    o[2 * h] = pack_bf16(lo.x * s, lo.y * s);
    o[2 * h + 1] = pack_bf16(hi.x * s, hi.y * s);
  }
  *reinterpret_cast<uint4*>(tile + swz(r, c0 + C)) = uint4{o[0], o[1], o[2], o[3]};
}

template <int LAYOUT>
__device__ __forceinline__ void decode_block_to_lds(const BlockRaw& b, char* tile, int r, int c0) {
  decode_chunk_to_lds<LAYOUT, 0>(b, tile, r, c0);
  decode_chunk_to_lds<LAYOUT, 1>(b, tile, r, c0);
  decode_chunk_to_lds<LAYOUT, 2>(b, tile, r, c0);
  decode_chunk_to_lds<LAYOUT, 3>(b, tile, r, c0);
}

template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint8_t* __restrict__ w, int n,
                                                        int nb, const uint16_t* __restrict__ a,
                                                        int m, int64_t lda,
                                                        uint16_t* __restrict__ c, int64_t ldc,
                                                        int m_tiles) {
  constexpr int BB = block_bytes(LAYOUT);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // Buffer b of the A tile at smem + 2b * kTileBytes, of the W tile one tile later.
  auto a_tile = [&](int b) { return smem + 2 * b * kTileBytes; };
  auto w_tile = [&](int b) { return smem + (2 * b + 1) * kTileBytes; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 1;  // 0..3: 64-row slab of the tile
  const int wn = wid & 1;   // 0..1: 128-column slab
  const int tile_id = blockIdx.x;
  const int m0 = (tile_id % m_tiles) * BM;
  const int n0 = (tile_id / m_tiles) * BN;
  const int64_t rowbytes = static_cast<int64_t>(nb) * BB;
  const int steps = nb / 2;  // BK = 64 = two blocks

  // A loader: thread -> 16-byte chunk (t % 8) of rows t/8 + 64 i, i = 0..3 (eight
  // threads cover a row's 128 contiguous bytes); staged in registers, written to the
  // swizzled LDS tile after the MFMAs of the current step.
  const int a_row0 = tid >> 3;
  const int a_chunk = tid & 7;
  struct AChunks {
    uint4 v0, v1, v2, v3;
  };
  const uint16_t* a_col = a + a_chunk * 8;
  auto a_row_ptr = [&](int i) { return a_col + min(m0 + a_row0 + 64 * i, m - 1) * lda; };
  // Rows past m are clamped to row m - 1; their results are never stored.
  const uint16_t* a_p0 = a_row_ptr(0);
  const uint16_t* a_p1 = a_row_ptr(1);
  const uint16_t* a_p2 = a_row_ptr(2);
  const uint16_t* a_p3 = a_row_ptr(3);
  auto load_a = [&](int s) {
    AChunks r;
    r.v0 = *reinterpret_cast<const uint4*>(a_p0 + s * BK);
    r.v1 = *reinterpret_cast<const uint4*>(a_p1 + s * BK);
    r.v2 = *reinterpret_cast<const uint4*>(a_p2 + s * BK);
    r.v3 = *reinterpret_cast<const uint4*>(a_p3 + s * BK);
    return r;
  };
  auto store_a = [&](const AChunks& r, char* tile) {
    *reinterpret_cast<uint4*>(tile + swz(a_row0, a_chunk)) = r.v0;
    *reinterpret_cast<uint4*>(tile + swz(a_row0 + 64, a_chunk)) = r.v1;
    *reinterpret_cast<uint4*>(tile + swz(a_row0 + 128, a_chunk)) = r.v2;
    *reinterpret_cast<uint4*>(tile + swz(a_row0 + 192, a_chunk)) = r.v3;
  };
  // W loader: thread -> (weight row, block of the step).
  const int w_r = tid >> 1;
  const int w_blk = tid & 1;
  const uint8_t* w_row = w + min(n0 + w_r, n - 1) * rowbytes + w_blk * BB;
  auto load_w = [&](int s) { return load_block<LAYOUT>(w_row + s * 2 * BB); };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Prologue: stage 0 in LDS, the weights of stage 1 in registers.
  {
    const AChunks a0 = load_a(0);
    const BlockRaw b0 = load_w(0);
    store_a(a0, a_tile(0));
    decode_block_to_lds<LAYOUT>(b0, w_tile(0), w_r, 4 * w_blk);
  }
  BlockRaw w_next = load_w(min(1, steps - 1));
  __syncthreads();

  const int fr = lane & 31;  // fragment row within a 32-row MFMA tile
  const int fk = lane >> 5;  // which 8-column half of a 16-column k slice
  // Branch-free main loop: on the last step the prefetches below are clamped to the
  // last stage and only refill the buffer that is no longer read.
  for (int s = 0; s < steps; ++s) {
    const int cur = s & 1;
    // Issue order matters: the A loads first and the weight loads after them, so that
    // storing A at the end of the step waits only for the A loads (vmcnt counts in issue
    // order); the scheduling barrier keeps the compiler from sinking the loads.
    const AChunks a_next = load_a(min(s + 1, steps - 1));
    const BlockRaw w_after = load_w(min(s + 2, steps - 1));  // two steps ahead
    __builtin_amdgcn_sched_barrier(0);
    const char* at = a_tile(cur);
    const char* wt = w_tile(cur);
    char* wn_tile = w_tile(cur ^ 1);
    bf16x8 af[2][2], bfr[2][4];
    auto load_frags = [&](int kk, int slot) {
      const int ck = 2 * kk + fk;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[slot][i] = *reinterpret_cast<const bf16x8*>(at + swz(wm * 64 + i * 32 + fr, ck));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[slot][j] = *reinterpret_cast<const bf16x8*>(wt + swz(wn * 128 + j * 32 + fr, ck));
    };
    auto mfmas = [&](int slot) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[slot][i], bfr[slot][j], acc[i][j], 0, 0, 0);
    };
    // k slice kk: fragments of kk+1 are read while the MFMAs of kk run, and one
    // 16-byte chunk of the next stage's weights is decoded alongside.
    load_frags(0, 0);
    load_frags(1, 1);
    mfmas(0);
    decode_chunk_to_lds<LAYOUT, 0>(w_next, wn_tile, w_r, 4 * w_blk);
    load_frags(2, 0);
    mfmas(1);
    decode_chunk_to_lds<LAYOUT, 1>(w_next, wn_tile, w_r, 4 * w_blk);
    load_frags(3, 1);
    mfmas(0);
    decode_chunk_to_lds<LAYOUT, 2>(w_next, wn_tile, w_r, 4 * w_blk);
    mfmas(1);
    decode_chunk_to_lds<LAYOUT, 3>(w_next, wn_tile, w_r, 4 * w_blk);
    __builtin_amdgcn_sched_barrier(0);
    store_a(a_next, a_tile(cur ^ 1));
    w_next = w_after;
    __syncthreads();
  }

  // Epilogue. 32x32 accumulator layout: register e of lane l holds row
  // 8*(e/4) + 4*(l/32) + (e%4), column l%32 of the MFMA tile.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + wn * 128 + j * 32 + (lane & 31);
      if (gn >= n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gm = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (gm < m) c[gm * ldc + gn] = bf16_rne(acc[i][j][e]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* w, int layout, int64_t n, int64_t k, const uint16_t* a,
                       int64_t m, int64_t lda, uint16_t* c, int64_t ldc, hipStream_t stream) {
  const int nb = static_cast<int>(k / 32);
  const size_t shm = 4 * static_cast<size_t>(kTileBytes);  // 128 KB
  // The dynamic-LDS limit is raised once per device and layout; threads that race
  // repeat the same idempotent call.
  static std::atomic<bool> attr_set[64][2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !attr_set[dev][layout].load(std::memory_order_acquire)) {
    const void* fn = layout == kDual ? reinterpret_cast<const void*>(&gemm_kernel<kDual>)
                                     : reinterpret_cast<const void*>(&gemm_kernel<kFast>);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm));
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev][layout].store(true, std::memory_order_release);
  }
  const int64_t n_tiles = (n + BN - 1) / BN;
  // Launch in chunks of whole M-tile groups so the grid stays within 2^31 workgroups.
  const int64_t max_m = int64_t(1) << 20;
  for (int64_t m_off = 0; m_off < m; m_off += max_m) {
    const int64_t mc = (m - m_off < max_m) ? (m - m_off) : max_m;
    const int m_tiles = static_cast<int>((mc + BM - 1) / BM);
    const dim3 grid(static_cast<unsigned>(m_tiles * n_tiles));
    const uint16_t* ap = a + m_off * lda;
    uint16_t* cp = c + m_off * ldc;
    if (layout == kDual)
      gemm_kernel<kDual><<<grid, dim3(kThreads), shm, stream>>>(w, static_cast<int>(n), nb, ap,
                                                                static_cast<int>(mc), lda, cp, ldc, m_tiles);
    else
      gemm_kernel<kFast><<<grid, dim3(kThreads), shm, stream>>>(w, static_cast<int>(n), nb, ap,
                                                                static_cast<int>(mc), lda, cp, ldc, m_tiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rfp4
