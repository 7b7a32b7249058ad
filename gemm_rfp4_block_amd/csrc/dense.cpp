// Dense bf16 GEMM for the dequantize-then-multiply prefill path (the variant the page
// lists next to the fused w4a16_gemm, "Feasibility Report: Porting ROCmFP4 to Atlas",
// "Kernel System"): C = A W^T with W already expanded to bf16, computed by rocBLAS.
// rocBLAS is opened with dlopen at first use, so the library has no link-time
// dependency on it; without it the call reports RFP4_ERR_UNSUPPORTED.
//
// Row-major C (m x n) = A (m x k) W^T (W n x k) is, read column-major, the product
// C' (n x m) = W' ^T A' with W' (k x n, leading dimension ldw) and A' (k x m, lda):
// rocBLAS "TN" with sizes (n, m, k).

#include <dlfcn.h>
#include <rocblas/rocblas.h>  // types and prototypes only

#include <mutex>

#include "rfp4.h"
#include "rfp4_internal.h"

namespace rfp4 {
namespace {

struct RocblasApi {
  decltype(&rocblas_create_handle) create = nullptr;
  decltype(&rocblas_set_stream) set_stream = nullptr;
  decltype(&rocblas_gemm_ex_64) gemm = nullptr;
  bool ok = false;
};

RocblasApi& rocblas_api() {
  static RocblasApi api;
  static std::once_flag once;
  std::call_once(once, [] {
    void* h = dlopen("librocblas.so.5", RTLD_NOW | RTLD_LOCAL);
    if (h == nullptr) h = dlopen("librocblas.so", RTLD_NOW | RTLD_LOCAL);
    if (h == nullptr) return;
    api.create = reinterpret_cast<decltype(api.create)>(dlsym(h, "rocblas_create_handle"));
    api.set_stream = reinterpret_cast<decltype(api.set_stream)>(dlsym(h, "rocblas_set_stream"));
    api.gemm = reinterpret_cast<decltype(api.gemm)>(dlsym(h, "rocblas_gemm_ex_64"));
    api.ok = api.create != nullptr && api.set_stream != nullptr && api.gemm != nullptr;
  });
  return api;
}

}  // namespace

int dense_gemm_bf16(const uint16_t* wb, int64_t n, int64_t k, int64_t ldw, const uint16_t* a,
                    int64_t m, int64_t lda, uint16_t* c, int64_t ldc, hipStream_t stream) {
  RocblasApi& api = rocblas_api();
  if (!api.ok) return RFP4_ERR_UNSUPPORTED;
  // One handle per (device, stream), created on first use and kept; the mutex covers
  // the handle table and the enqueue (rocBLAS handles are not shared between threads).
  struct Entry {
    int dev;
    hipStream_t stream;
    rocblas_handle handle;
  };
  static std::mutex mu;
  static Entry entries[256];
  static int count = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RFP4_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  rocblas_handle h = nullptr;
  for (int i = 0; i < count; ++i)
    if (entries[i].dev == dev && entries[i].stream == stream) h = entries[i].handle;
  if (h == nullptr) {
    if (count == 256) return RFP4_ERR_HIP;
    if (api.create(&h) != rocblas_status_success) return RFP4_ERR_HIP;
    if (api.set_stream(h, stream) != rocblas_status_success) return RFP4_ERR_HIP;
    entries[count++] = Entry{dev, stream, h};
  }
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_status st =
      api.gemm(h, rocblas_operation_transpose, rocblas_operation_none, n, m, k, &alpha, wb,
               rocblas_datatype_bf16_r, ldw, a, rocblas_datatype_bf16_r, lda, &beta, c,
               rocblas_datatype_bf16_r, ldc, c, rocblas_datatype_bf16_r, ldc,
               rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? RFP4_OK : RFP4_ERR_HIP;
}

}  // namespace rfp4
