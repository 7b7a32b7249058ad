// Host entry of the fused dequant + GEMV (kernels and launch plans in gemv_impl.h,
// compiled once per activation dtype in gemv_f16.hip and gemv_bf16.hip).

#include "rfp4_internal.h"

namespace rfp4 {

// CU count of the current device, queried once per device and kept in an atomic
// cache (threads that race store the same value).
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

hipError_t launch_gemv(const GemvPart* parts, int count, int layout, int64_t k, const void* x,
                       int xdtype, int batch, int64_t ldx, hipStream_t stream) {
  const int nb = static_cast<int>(k / 32);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  return xdtype == kF16 ? launch_gemv_f16(parts, count, layout, nb, xp, batch, ldx, stream)
                        : launch_gemv_bf16(parts, count, layout, nb, xp, batch, ldx, stream);
}

}  // namespace rfp4
