// Host entry of the fused dequant + GEMV (kernels and launch plans in gemv_impl.h,
// compiled once per activation dtype in gemv_f16.hip and gemv_bf16.hip).

#include <mutex>
#include <vector>

#include "rfp4_internal.h"

namespace rfp4 {

// Device workspaces, one per (kind, device, stream): calls ordered on a stream reuse
// theirs and calls on different streams never share one. Nothing here frees memory or
// synchronizes: a launch that needs more than its stream's workspace holds gets a new
// buffer (at least twice as large), and the outgrown one stays allocated, unused, until
// the process ends, because kernels still in flight or graphs captured earlier may
// write to it. Growth by doubling bounds what is kept to the size of the live buffer.
// Nothing is allocated while the stream is being captured.
hipError_t stream_workspace(int kind, hipStream_t stream, size_t bytes, bool zero, void** out) {
  struct Entry {
    int kind;
    int dev;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
  };
  static std::mutex mu;
  static std::vector<Entry> entries;  // live workspaces
  static std::vector<void*> retired;  // outgrown workspaces, never freed
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  Entry* en = nullptr;
  for (Entry& x : entries)
    if (x.kind == kind && x.dev == dev && x.stream == stream) en = &x;
  if (en != nullptr && en->bytes >= bytes) {
    *out = en->ptr;
    return hipSuccess;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return e;
  if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
  size_t want = bytes;
  if (en != nullptr && want < 2 * en->bytes) want = 2 * en->bytes;
  void* p = nullptr;
  e = hipMalloc(&p, want);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // the failed allocation's error is reported here, not later
    return e;
  }
  if (zero) {
    e = hipMemsetAsync(p, 0, want, stream);
    if (e != hipSuccess) {
      retired.push_back(p);
      return e;
    }
  }
  if (en == nullptr) {
    entries.push_back(Entry{kind, dev, stream, p, want});
  } else {
    retired.push_back(en->ptr);
    en->ptr = p;
    en->bytes = want;
  }
  *out = p;
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
                       int xdtype, int batch, int64_t ldx, const Force& force, hipStream_t stream) {
  const int nb = static_cast<int>(k / 32);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  return xdtype == kF16 ? launch_gemv_f16(parts, count, layout, nb, xp, batch, ldx, force, stream)
                        : launch_gemv_bf16(parts, count, layout, nb, xp, batch, ldx, force, stream);
}

}  // namespace rfp4
