// librfp4_bench.so: a plain streaming read of device memory (the HBM read ceiling the
// decode GEMV is measured against) and a dense bf16 matrix-core loop (the sustained
// MFMA rate the prefill GEMM is measured against). Declared in include/rfp4_bench.h.

#include <hip/hip_runtime.h>

#include "rfp4_bench.h"

namespace {

constexpr int kThreads = 256;

// Workgroup w reads runs of kThreads * U 16-byte pieces (consecutive threads read
// consecutive pieces, so a wavefront's load covers 1 KiB), runs w, w + grid, ...
template <int U>
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ p, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t run = static_cast<size_t>(kThreads) * U;
  for (size_t base = blockIdx.x * run; base < n16; base += gridDim.x * run) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + u * kThreads + threadIdx.x;
      v[u] = i < n16 ? p[i] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // The data never XORs to this value in the measured buffers' construction, and if it
  // did one word is written: the loads are kept without a store per thread.
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// A hash of the lane, workgroup and operand index to a value in [-1, 1): operands whose
// bits differ from one instruction to the next, as in a real product (constant operands
// draw less power and run faster).
__device__ inline float hash_unit(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return static_cast<float>(x & 0xFFFFFFu) / 8388608.0f - 1.0f;
}

// Every wavefront issues iters x 8 v_mfma_f32_32x32x16_bf16 into 8 independent
// accumulators, cycling through 4 A and 4 B operands; nothing else in the loop.
__global__ __launch_bounds__(512) void mfma_kernel(int iters, uint32_t* __restrict__ sink) {
  bf16x8 a[4], b[4];
  const uint32_t id = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[q][i] = static_cast<__bf16>(hash_unit(id * 131u + q * 17u + i));
      b[q][i] = static_cast<__bf16>(hash_unit(id * 71u + q * 29u + i * 3u + 100003u));
    }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j + (j >> 2)) & 3], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (__float_as_uint(s) == 0x7FC0FFEEu) sink[0] = 1u;  // a NaN payload the sums never take
}

}  // namespace

extern "C" int rfp4bench_mfma(int wgs_per_cu, int threads, int iters, uint32_t* sink, void* stream) {
  if (sink == nullptr || wgs_per_cu < 1 || wgs_per_cu > 8 || iters < 1) return -1;
  if (threads != 64 && threads != 128 && threads != 256 && threads != 512) return -1;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return static_cast<int>(e);
  mfma_kernel<<<dim3(static_cast<unsigned>(cus * wgs_per_cu)), dim3(threads), 0, static_cast<hipStream_t>(stream)>>>(
      iters, sink);
  return static_cast<int>(hipGetLastError());
}

extern "C" int rfp4bench_read(const void* p, size_t bytes, int unroll, int wgs_per_cu, uint32_t* sink,
                              void* stream) {
  if (p == nullptr || sink == nullptr || bytes == 0 || (bytes % 16) != 0 ||
      (reinterpret_cast<uintptr_t>(p) & 15u) != 0)
    return -1;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return -1;
  if (wgs_per_cu < 1 || wgs_per_cu > 32) return -1;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return static_cast<int>(e);
  const size_t n16 = bytes / 16;
  const dim3 grid(static_cast<unsigned>(cus * wgs_per_cu)), block(kThreads);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* q = static_cast<const uint4*>(p);
  switch (unroll) {
    case 1: read_kernel<1><<<grid, block, 0, s>>>(q, n16, sink); break;
    case 2: read_kernel<2><<<grid, block, 0, s>>>(q, n16, sink); break;
    case 4: read_kernel<4><<<grid, block, 0, s>>>(q, n16, sink); break;
    default: read_kernel<8><<<grid, block, 0, s>>>(q, n16, sink); break;
  }
  return static_cast<int>(hipGetLastError());
}
