// Standalone dequantization: packed ROCmFP4 rows -> fp32 or bf16 matrix, bit-exact.
//
// The page's "reference decoder" ("Feasibility Report: Porting ROCmFP4 to Atlas",
// "Integration Options", Option 1). Write-bound: 4 bytes out per 0.53-0.56 bytes in.
//
// Mapping (fp32): eight consecutive threads own one block; thread s (0..7) produces weights
// 4s .. 4s+3 and writes them as one 16-byte store, so a wavefront writes 1 KB of
// contiguous output per instruction. Threads 0..3 decode the low nibbles of qs
// bytes 4s..4s+3 (first half), threads 4..7 the high nibbles of qs bytes
// 4(s-4)..4(s-4)+3 (second half).

#include "rfp4_decode.h"
#include "rfp4_internal.h"

// Output stores are non-temporal (the output is written once and not read back by this
// kernel): measured on the up-projection matrix, fp32 out 83.6 -> 56.9 us (4.9 -> 7.2 TB/s),
// bf16 out 34.5 -> 33.4 us. RFP4_DEQUANT_NT=0 builds ordinary stores.
#ifndef RFP4_DEQUANT_NT
#define RFP4_DEQUANT_NT 1
#endif

namespace rfp4 {
namespace {

template <int LAYOUT, bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ w, int64_t nb,
                                                      int64_t total_threads, void* __restrict__ out,
                                                      int64_t ldo) {
  constexpr int BB = block_bytes(LAYOUT);
  constexpr int TPB = BF16 ? 4 : 8;  // threads per block
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total_threads;
       g += stride) {
    const int64_t blk = g / TPB;  // flat block index, rows back to back
    const int s = static_cast<int>(g % TPB);
    const int64_t row = blk / nb;
    const int64_t j = blk - row * nb;
    const uint8_t* p = w + blk * BB;
    if constexpr (!BF16) {
      const uint32_t q = load4(p + 4 * (s & 3));
      const uint32_t sb = p[16 + ((LAYOUT == kDual) ? (s >> 2) : 0)];
      const uint32_t codes = (s < 4) ? codes_low_exact(q) : codes_high_exact(q);
      const f32x2 a = pair_f32(codes, false);
      const f32x2 b = pair_f32(codes, true);
      const float sc = scale_exact(sb);
      float4 v;
      v.x = a.x * sc;
      v.y = a.y * sc;
      v.z = b.x * sc;
      v.w = b.y * sc;
      float4* const dst = reinterpret_cast<float4*>(static_cast<float*>(out) + row * ldo + j * 32 + 4 * s);
#if RFP4_DEQUANT_NT
      typedef float nt4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(nt4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt4*>(dst));
#else
      *dst = v;
#endif
    } else {
      // Thread s writes weights 8s .. 8s+7: the low (s < 2) or high (s >= 2) nibbles of
      // qs bytes 8(s % 2) .. 8(s % 2) + 7. Every value is a bf16 value, so keeping the
      // upper 16 bits of the fp32 product is exact.
      const int plane = s >> 1;
      const uint32_t q0 = load4(p + 8 * (s & 1));
      const uint32_t q1 = load4(p + 8 * (s & 1) + 4);
      const uint32_t sb = p[16 + ((LAYOUT == kDual) ? plane : 0)];
      const float sc = scale_exact(sb);
      const uint32_t c0 = plane ? codes_high_exact(q0) : codes_low_exact(q0);
      const uint32_t c1 = plane ? codes_high_exact(q1) : codes_low_exact(q1);
      const f32x2 v[4] = {pair_f32(c0, false), pair_f32(c0, true), pair_f32(c1, false), pair_f32(c1, true)};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = (__float_as_uint(v[i].x * sc) >> 16) | (__float_as_uint(v[i].y * sc) & 0xFFFF0000u);
      uint4* const dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + row * ldo + j * 32 + 8 * s);
#if RFP4_DEQUANT_NT
      typedef uint32_t ntu4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(ntu4{o[0], o[1], o[2], o[3]}, reinterpret_cast<ntu4*>(dst));
#else
      *dst = uint4{o[0], o[1], o[2], o[3]};
#endif
    }
  }
}

template <bool BF16>
hipError_t launch_dequant_t(const uint8_t* w, int layout, int64_t n, int64_t k, void* out,
                            int64_t ldo, hipStream_t stream) {
  const int64_t nb = k / 32;
  const int64_t total = n * nb * (BF16 ? 4 : 8);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  if (layout == kDual)
    dequant_kernel<kDual, BF16><<<dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream>>>(
        w, nb, total, out, ldo);
  else
    dequant_kernel<kFast, BF16><<<dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream>>>(
        w, nb, total, out, ldo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint8_t* w, int layout, int64_t n, int64_t k, float* out,
                          int64_t ldo, hipStream_t stream) {
  return launch_dequant_t<false>(w, layout, n, k, out, ldo, stream);
}

hipError_t launch_dequant_bf16(const uint8_t* w, int layout, int64_t n, int64_t k, uint16_t* out,
                               int64_t ldo, hipStream_t stream) {
  return launch_dequant_t<true>(w, layout, n, k, out, ldo, stream);
}

}  // namespace rfp4
