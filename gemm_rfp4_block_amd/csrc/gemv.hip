// Fused dequant + GEMV for decode: y[b][r] = sum_c W[r][c] * x[b][c], batch 1..8.
//
// The page names gemv as the decode hot path ("Feasibility Report: Porting ROCmFP4
// to Atlas", "Kernel System" and "Integration Options", Option 2) and says that on
// AMD the bottleneck is memory bandwidth ("Why AMD is Different from NVIDIA"). The
// kernel therefore reads every packed block exactly once from HBM and does all the
// decode in registers.
//
// Work mapping. A wavefront covers RL rows x CL column lanes (RL * CL = 64, CL =
// gcd(64, blocks per row)), so every lane owns the same number of blocks of its row
// and lanes of one row read adjacent blocks (a run of CL * 18 or CL * 17 contiguous
// bytes per load instruction). Each lane loads a block's 16 index bytes with one
// unaligned 16-byte load and its scale byte(s) with one small load, decodes the 32
// weights to f16/bf16 pairs (see rfp4_decode.h) and multiplies them with the
// activations with v_dot2_f32_{f16,bf16}: one fp32 partial sum per 16-weight half,
// then one fp32 FMA with that half's E4M3 scale. The partial sums of the CL lanes of
// a row are combined with a butterfly of cross-lane shuffles, and the final 1/2 of
// the half-scale is applied at the store.
//
// Activations: staged once per workgroup into LDS when batch * k * 2 bytes fits the
// budget, in 16-byte units ordered [batch][chunk of 8 values][block] so that the 64
// lanes of a wavefront read consecutive 16-byte units (no bank conflicts); otherwise
// read straight from global memory (they stay cache-resident).

#include "rfp4_decode.h"
#include "rfp4_internal.h"

namespace rfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kXLdsBudget = 40 * 1024;

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

template <int LAYOUT, int XT, int BATCH, bool XLDS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t* __restrict__ w, int n,
                                                        int nb, int log2cl, int groups,
                                                        const uint16_t* __restrict__ x,
                                                        int64_t ldx, float* __restrict__ y,
                                                        int64_t ldy) {
  typedef Act<XT> A;
  typedef typename A::pair pair;
  constexpr int BB = block_bytes(LAYOUT);
  extern __shared__ uint4 xs[];

  if constexpr (XLDS) {
    const int units = BATCH * 4 * nb;
    for (int u = threadIdx.x; u < units; u += kThreads) {
      const int j = u % nb;
      const int bc = u / nb;
      xs[u] = *reinterpret_cast<const uint4*>(x + (bc >> 2) * ldx + 32 * j + 8 * (bc & 3));
    }
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int cl = 1 << log2cl;
  const int rl = 64 >> log2cl;
  const int r_in = lane >> log2cl;
  const int c = lane & (cl - 1);
  const int iters = nb >> log2cl;
  const int wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (kThreads / 64);
  const int64_t rowbytes = static_cast<int64_t>(nb) * BB;

  for (int g = wave; g < groups; g += nwaves) {
    const int row = g * rl + r_in;
    float acc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) acc[b] = 0.f;
    if (row < n) {
      const uint8_t* prow = w + row * rowbytes;
#pragma unroll 2
      for (int i = 0; i < iters; ++i) {
        const int j = c + (i << log2cl);
        const uint8_t* p = prow + j * BB;
        const uint4 qv = load16(p);
        uint32_t sw;
        if constexpr (LAYOUT == kDual) {
          uint16_t s2;
          __builtin_memcpy(&s2, p + 16, 2);
          sw = s2 & 0x7F7Fu;
        } else {
          sw = p[16] & 0x7Fu;
        }
        const uint32_t q[4] = {qv.x, qv.y, qv.z, qv.w};
        pair wl[8], wh[8];  // first half (low nibbles), second half (high nibbles)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t lo = codes_low(q[d]);
          const uint32_t hi = codes_high(q[d]);
          wl[2 * d] = A::decode(lo, false);
          wl[2 * d + 1] = A::decode(lo, true);
          wh[2 * d] = A::decode(hi, false);
          wh[2 * d + 1] = A::decode(hi, true);
        }
        const float s0 = e4m3_hw<0>(sw);
        const float s1 = (LAYOUT == kDual) ? e4m3_hw<1>(sw) : s0;
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          uint4 xc[4];
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            if constexpr (XLDS)
              xc[cc] = xs[(b * 4 + cc) * nb + j];
            else
              xc[cc] = *reinterpret_cast<const uint4*>(x + b * ldx + 32 * j + 8 * cc);
          }
          const uint32_t x0[8] = {xc[0].x, xc[0].y, xc[0].z, xc[0].w,
                                  xc[1].x, xc[1].y, xc[1].z, xc[1].w};
          const uint32_t x1[8] = {xc[2].x, xc[2].y, xc[2].z, xc[2].w,
                                  xc[3].x, xc[3].y, xc[3].z, xc[3].w};
          float p0 = 0.f, p1 = 0.f;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            p0 = A::dot(wl[t], x0[t], p0);
            p1 = A::dot(wh[t], x1[t], p1);
          }
          acc[b] = __builtin_fmaf(s0, p0, acc[b]);
          acc[b] = __builtin_fmaf(s1, p1, acc[b]);
        }
      }
    }
    for (int off = cl >> 1; off >= 1; off >>= 1) {
#pragma unroll
      for (int b = 0; b < BATCH; ++b) acc[b] += __shfl_xor(acc[b], off, 64);
    }
    if (c == 0 && row < n) {
#pragma unroll
      for (int b = 0; b < BATCH; ++b) y[b * ldy + row] = 0.5f * acc[b];
    }
  }
}

int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

template <int LAYOUT, int XT, int BATCH>
hipError_t launch3(const uint8_t* w, int n, int nb, const uint16_t* x, int64_t ldx, float* y,
                   int64_t ldy, hipStream_t stream) {
  int g = 64;
  while (nb % g) g >>= 1;  // CL = gcd(64, nb); nb is a multiple of 8
  int log2cl = 0;
  while ((1 << log2cl) < g) ++log2cl;
  const int rl = 64 >> log2cl;
  const int groups = (n + rl - 1) / rl;
  const int waves_per_wg = kThreads / 64;
  int wgs = (groups + waves_per_wg - 1) / waves_per_wg;
  const int cap = device_cu_count() * 8;
  if (wgs > cap) wgs = cap;
  const size_t xbytes = static_cast<size_t>(BATCH) * nb * 32 * 2;
  if (xbytes <= static_cast<size_t>(kXLdsBudget)) {
    gemv_kernel<LAYOUT, XT, BATCH, true><<<dim3(wgs), dim3(kThreads), xbytes, stream>>>(
        w, n, nb, log2cl, groups, x, ldx, y, ldy);
  } else {
    gemv_kernel<LAYOUT, XT, BATCH, false><<<dim3(wgs), dim3(kThreads), 0, stream>>>(
        w, n, nb, log2cl, groups, x, ldx, y, ldy);
  }
  return hipGetLastError();
}

template <int LAYOUT, int XT>
hipError_t launch2(const uint8_t* w, int n, int nb, const uint16_t* x, int batch, int64_t ldx,
                   float* y, int64_t ldy, hipStream_t s) {
  switch (batch) {
    case 1: return launch3<LAYOUT, XT, 1>(w, n, nb, x, ldx, y, ldy, s);
    case 2: return launch3<LAYOUT, XT, 2>(w, n, nb, x, ldx, y, ldy, s);
    case 3: return launch3<LAYOUT, XT, 3>(w, n, nb, x, ldx, y, ldy, s);
    case 4: return launch3<LAYOUT, XT, 4>(w, n, nb, x, ldx, y, ldy, s);
    case 5: return launch3<LAYOUT, XT, 5>(w, n, nb, x, ldx, y, ldy, s);
    case 6: return launch3<LAYOUT, XT, 6>(w, n, nb, x, ldx, y, ldy, s);
    case 7: return launch3<LAYOUT, XT, 7>(w, n, nb, x, ldx, y, ldy, s);
    default: return launch3<LAYOUT, XT, 8>(w, n, nb, x, ldx, y, ldy, s);
  }
}

}  // namespace

hipError_t launch_gemv(const uint8_t* w, int layout, int64_t n, int64_t k, const void* x,
                       int xdtype, int batch, int64_t ldx, float* y, int64_t ldy,
                       hipStream_t stream) {
  const int nb = static_cast<int>(k / 32);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const int ni = static_cast<int>(n);
  if (layout == kDual) {
    return xdtype == kF16 ? launch2<kDual, kF16>(w, ni, nb, xp, batch, ldx, y, ldy, stream)
                          : launch2<kDual, kBF16>(w, ni, nb, xp, batch, ldx, y, ldy, stream);
  }
  return xdtype == kF16 ? launch2<kFast, kF16>(w, ni, nb, xp, batch, ldx, y, ldy, stream)
                        : launch2<kFast, kBF16>(w, ni, nb, xp, batch, ldx, y, ldy, stream);
}

}  // namespace rfp4
