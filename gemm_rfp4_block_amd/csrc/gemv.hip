// Host entry of the fused dequant + GEMV (kernels and launch plans in gemv_impl.h,
// compiled once per activation dtype in gemv_f16.hip and gemv_bf16.hip).

#include <mutex>

#include "rfp4_internal.h"

namespace rfp4 {

// Device workspaces, one per (kind, device, stream): calls ordered on a stream reuse
// theirs and calls on different streams never share one. A workspace grows on demand
// (after the stream's earlier work has finished), starts zero-filled and is kept until
// the process ends. Nothing is allocated while the stream is being captured.
hipError_t stream_workspace(int kind, hipStream_t stream, size_t bytes, void** out) {
  struct Entry {
    int kind;
    int dev;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
  };
  static std::mutex mu;
  static Entry entries[256];
  static int count = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  Entry* en = nullptr;
  for (int i = 0; i < count; ++i)
    if (entries[i].kind == kind && entries[i].dev == dev && entries[i].stream == stream) en = &entries[i];
  if (en == nullptr) {
    if (count == 256) return hipErrorOutOfMemory;
    en = &entries[count++];
    *en = Entry{kind, dev, stream, nullptr, 0};
  }
  if (en->bytes < bytes) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    if (en->ptr != nullptr) {
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return e;
      e = hipFree(en->ptr);
      en->ptr = nullptr;
      en->bytes = 0;
      if (e != hipSuccess) return e;
    }
    e = hipMalloc(&en->ptr, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // the failed allocation's error is reported here, not later
      en->ptr = nullptr;
      return e;
    }
    e = hipMemsetAsync(en->ptr, 0, bytes, stream);
    if (e != hipSuccess) return e;
    en->bytes = bytes;
  }
  *out = en->ptr;
  return hipSuccess;
}

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
