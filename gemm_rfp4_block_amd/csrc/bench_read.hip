// librfp4_bench.so: a plain streaming read of device memory (the HBM read ceiling the
// decode GEMV is measured against). Declared in include/rfp4_bench.h.

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

}  // namespace

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
