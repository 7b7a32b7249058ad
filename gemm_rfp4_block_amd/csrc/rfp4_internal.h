// Internal declarations shared by the host API and the kernel translation units of
// librfp4.so. Not part of the public ABI (see include/rfp4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "rfp4.h"

namespace rfp4 {

constexpr int kDual = 0;
constexpr int kFast = 1;
constexpr int kF16 = 0;
constexpr int kBF16 = 1;
constexpr int kF32 = 2;

// Bytes per 32-weight block ("Block Layout": qs[16] then e[2] or e).
constexpr int block_bytes(int layout) { return layout == kDual ? 18 : 17; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Per-(kind, device, stream) device workspace of at least `bytes`, kept until the
// process ends. A workspace is never freed and nothing synchronizes: when a launch needs
// more than the stream has, a new buffer of at least twice the old size is allocated
// and the old one is kept, unused (a graph captured earlier may still write to it).
// A new buffer is zero-filled (an asynchronous fill ordered on the stream) when
// `zero` is set. hipErrorStreamCaptureUnsupported while the stream is being captured
// and its workspace is too small (nothing is allocated during a capture).
constexpr int kWorkspaceGemm = 0;  // k-split partial tiles of rfp4_gemm
constexpr int kWorkspaceGemv = 1;  // split-chunk partial sums and arrival counters of rfp4_gemv
hipError_t stream_workspace(int kind, hipStream_t stream, size_t bytes, bool zero, void** out);

// The kernel and plan overrides of the _ex entry points (rfp4_force in rfp4.h), checked
// by the API layer; a zero-filled struct is the default behaviour.
typedef rfp4_force Force;

// Launchers. Arguments have been checked by the API layer: shapes in range, rows
// 16-byte aligned, pointers non-null and aligned as the public header requires.
hipError_t launch_dequant(const uint8_t* w, int layout, int64_t n, int64_t k, float* out,
                          int64_t ldo, hipStream_t stream);
// Encoder: n rows of k values (row stride lds elements, dtype kF32 / kBF16 / kF16)
// -> n * k / 32 packed blocks, back to back from `out` (16-byte aligned).
hipError_t launch_quantize(const void* src, int dtype, int64_t n, int64_t k, int64_t lds,
                           int layout, uint8_t* out, hipStream_t stream);
hipError_t launch_dequant_bf16(const uint8_t* w, int layout, int64_t n, int64_t k, uint16_t* out,
                               int64_t ldo, hipStream_t stream);

// Dense bf16 C = A W^T through rocBLAS (loaded at first use); RFP4 status codes:
// 0 = ok, RFP4_ERR_UNSUPPORTED when rocBLAS is unavailable, RFP4_ERR_HIP on failure.
int dense_gemm_bf16(const uint16_t* wb, int64_t n, int64_t k, int64_t ldw, const uint16_t* a,
                    int64_t m, int64_t lda, uint16_t* c, int64_t ldc, hipStream_t stream);

// One matrix of a GEMV launch: n rows of packed weights at w, outputs y[b * ldy + r].
constexpr int kMaxGemvParts = 8;
struct GemvPart {
  const uint8_t* w;
  int64_t n;
  float* y;
  int64_t ldy;
};

// 1 <= count <= kMaxGemvParts matrices sharing k and the activations.
hipError_t launch_gemv(const GemvPart* parts, int count, int layout, int64_t k, const void* x,
                       int xdtype, int batch, int64_t ldx, const Force& force, hipStream_t stream);
// The same for one activation dtype (nb = k / 32 blocks per row).
hipError_t launch_gemv_f16(const GemvPart* parts, int count, int layout, int nb, const uint16_t* x,
                           int batch, int64_t ldx, const Force& force, hipStream_t stream);
hipError_t launch_gemv_bf16(const GemvPart* parts, int count, int layout, int nb, const uint16_t* x,
                            int batch, int64_t ldx, const Force& force, hipStream_t stream);

hipError_t launch_gemm(const uint8_t* w, int layout, int64_t n, int64_t k, const uint16_t* a,
                       int64_t m, int64_t lda, uint16_t* c, int64_t ldc, const Force& force,
                       hipStream_t stream);

// The allocation-free GEMM: partial sums of split plans in a static device array of
// kGemmScratchBytes per GPU; plans are chosen among those that fit it, and a forced
// plan that needs more is rejected by the API layer (gemm_noalloc_plan_bytes).
constexpr size_t kGemmScratchBytes = RFP4_GEMM_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
double gemm_noalloc_plan_bytes(int64_t n, int64_t k, int64_t m, const Force& force);
hipError_t launch_gemm_noalloc(const uint8_t* w, int layout, int64_t n, int64_t k, const uint16_t* a,
                               int64_t m, int64_t lda, uint16_t* c, int64_t ldc, const Force& force,
                               hipStream_t stream);

}  // namespace rfp4
