// Weight-only 4-bit GEMM for prefill: C[m][r] = bf16( sum_c A[m][c] * W[r][c] ).
//
// The page names this kernel w4a16_gemm, a weight-only 4-bit GEMM for prefill
// ("Feasibility Report: Porting ROCmFP4 to Atlas", "Kernel System"). Prefill is a
// dense contraction, so it runs on the matrix cores: each workgroup decodes a tile
// of packed weights into LDS as bf16 (exact: every codebook value times every
// decoded scale is a bf16 value) and feeds v_mfma_f32_16x16x32_bf16 with fp32
// accumulation; the epilogue rounds to bf16 (nearest even).
//
// Tiling: a 256-thread workgroup owns a BM x BN tile of C; per step it stages a
// BM x 32 slice of A and the matching 32-column slice of BN weight rows (exactly one
// ROCmFP4 block per row) into LDS; each of the four wavefronts computes a 64 x 64
// sub-tile as 4 x 4 MFMA tiles of 16 x 16.

#include "rfp4_decode.h"
#include "rfp4_internal.h"

namespace rfp4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 32;
constexpr int LDSK = BK + 8;  // padded row length in bf16 (80 bytes)

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  // Both values are exactly representable in bf16, so truncation is exact.
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int LAYOUT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ w, int n, int nb,
                                                   const uint16_t* __restrict__ a, int m,
                                                   int64_t lda, uint16_t* __restrict__ c,
                                                   int64_t ldc) {
  constexpr int BB = block_bytes(LAYOUT);
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDSK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * LDSK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1;
  const int wn = wid & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int64_t rowbytes = static_cast<int64_t>(nb) * BB;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ld_row = tid >> 1;  // 0..127
  const int ld_part = tid & 1;  // which 16 columns of the 32

  for (int kb = 0; kb < nb; ++kb) {
    // A slice: row ld_row, columns 32*kb + 16*ld_part .. +16
    {
      const int gm = m0 + ld_row;
      uint4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
      if (gm < m) {
        const uint16_t* src = a + gm * lda + kb * BK + 16 * ld_part;
        v0 = *reinterpret_cast<const uint4*>(src);
        v1 = *reinterpret_cast<const uint4*>(src + 8);
      }
      uint4* dst = reinterpret_cast<uint4*>(As + ld_row * LDSK + 16 * ld_part);
      dst[0] = v0;
      dst[1] = v1;
    }
    // W slice: weight row ld_row, half ld_part of block kb, decoded to bf16.
    {
      const int gn = n0 + ld_row;
      uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (gn < n) {
        const uint8_t* p = w + gn * rowbytes + kb * BB;
        const uint4 qv = load16(p);
        const uint32_t sb = p[16 + ((LAYOUT == kDual) ? ld_part : 0)];
        const float s = scale_exact(sb);
        const uint32_t q[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t codes = ld_part ? codes_high(q[d]) : codes_low(q[d]);
          const f32x2 lo = pair_f32(codes, false);
          const f32x2 hi = pair_f32(codes, true);
          out[2 * d] = pack_bf16(lo.x * s, lo.y * s);
          out[2 * d + 1] = pack_bf16(hi.x * s, hi.y * s);
        }
      }
      uint4* dst = reinterpret_cast<uint4*>(Ws + ld_row * LDSK + 16 * ld_part);
      dst[0] = uint4{out[0], out[1], out[2], out[3]};
      dst[1] = uint4{out[4], out[5], out[6], out[7]};
    }
    __syncthreads();

    bf16x8 af[4], bfr[4];
    const int fr = lane & 15;
    const int fk = 8 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      af[t] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + t * 16 + fr) * LDSK + fk);
      bfr[t] = *reinterpret_cast<const bf16x8*>(Ws + (wn * 64 + t * 16 + fr) * LDSK + fk);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    __syncthreads();
  }

  // D layout of a 16x16 tile: lane holds rows 4*(lane/16) + e, column lane % 16.
  const int col_in = lane & 15;
  const int row_in = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + wn * 64 + j * 16 + col_in;
      if (gn >= n) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gm = m0 + wm * 64 + i * 16 + row_in + e;
        if (gm < m) c[gm * ldc + gn] = bf16_rne(acc[i][j][e]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* w, int layout, int64_t n, int64_t k, const uint16_t* a,
                       int64_t m, int64_t lda, uint16_t* c, int64_t ldc, hipStream_t stream) {
  const int nb = static_cast<int>(k / 32);
  const int64_t max_m = int64_t(65535) * BM;  // grid.y limit per launch
  for (int64_t m_off = 0; m_off < m; m_off += max_m) {
    const int64_t mc = (m - m_off < max_m) ? (m - m_off) : max_m;
    const dim3 grid(static_cast<unsigned>((n + BN - 1) / BN), static_cast<unsigned>((mc + BM - 1) / BM));
    const uint16_t* ap = a + m_off * lda;
    uint16_t* cp = c + m_off * ldc;
    if (layout == kDual)
      gemm_kernel<kDual><<<grid, dim3(256), 0, stream>>>(w, static_cast<int>(n), nb, ap,
                                                         static_cast<int>(mc), lda, cp, ldc);
    else
      gemm_kernel<kFast><<<grid, dim3(256), 0, stream>>>(w, static_cast<int>(n), nb, ap,
                                                         static_cast<int>(mc), lda, cp, ldc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rfp4
