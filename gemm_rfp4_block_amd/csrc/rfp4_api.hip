// Host side of librfp4.so: the C ABI declared in include/rfp4.h.
//
// Every argument is checked here, before any HIP call, so that argument errors are
// reported on machines without a GPU and never reach a kernel. The row validation of
// "Feasibility Report: Porting ROCmFP4 to Atlas", "Scale Format" (reject non-finite
// scale bytes at load time) runs on the host in rfp4_validate.

#include "rfp4.h"

#include <stdint.h>

#include "rfp4_internal.h"

namespace {

constexpr int64_t kMaxDim = 2147483647;  // n, m, k <= 2^31 - 1
static_assert(RFP4_MAX_GEMV_PARTS == rfp4::kMaxGemvParts, "parts limit of the header and the kernels");
static_assert(RFP4_F16 == rfp4::kF16 && RFP4_BF16 == rfp4::kBF16 && RFP4_F32 == rfp4::kF32,
              "dtype codes of the header and the kernels");
constexpr int64_t kMaxElems = int64_t(1) << 39;  // elements of A or C (2^40 bytes of bf16)

bool layout_ok(int layout) { return layout == RFP4_DUAL || layout == RFP4_FAST; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// Activations, A, y and C need only 4-byte alignment: the kernels store outputs one
// element at a time, and gfx950's global vector loads take any address (an activation
// row that is not 16-byte aligned costs load cycles, not correctness).
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shape and alignment of the packed weight matrix, shared by every device entry point.
// Rows may have any length (k % 32 == 0): the kernels read blocks at any byte offset.
rfp4_status check_weights(const void* w, int layout, int64_t n, int64_t k) {
  if (!layout_ok(layout)) return RFP4_ERR_UNSUPPORTED;
  if (n < 1 || n > kMaxDim || k < 32 || k > kMaxDim || (k % 32) != 0) return RFP4_ERR_SHAPE;
  if (w == nullptr) return RFP4_ERR_NULL;
  if (n * (k / 32) * rfp4::block_bytes(layout) > (int64_t(1) << 40)) return RFP4_ERR_SHAPE;
  if (!aligned16(w)) return RFP4_ERR_UNSUPPORTED;
  return RFP4_OK;
}

rfp4_status from_hip(hipError_t e) { return e == hipSuccess ? RFP4_OK : RFP4_ERR_HIP; }

// Copies `force` (NULL = all defaults) after checking every field against the values
// rfp4.h lists.
rfp4_status check_force(const rfp4_force* force, rfp4::Force* out) {
  *out = rfp4::Force{};
  if (force == nullptr) return RFP4_OK;
  const rfp4_force& f = *force;
  if (f.gemv_kernel < RFP4_GEMV_KERNEL_AUTO || f.gemv_kernel > RFP4_GEMV_KERNEL_NO_TALL) return RFP4_ERR_UNSUPPORTED;
  if (f.gemv_unit_blocks == 0) {
    if (f.gemv_lanes_per_row != 0) return RFP4_ERR_UNSUPPORTED;
  } else {
    const int cl = f.gemv_lanes_per_row;
    if (f.gemv_unit_blocks != 1 && f.gemv_unit_blocks != 2) return RFP4_ERR_UNSUPPORTED;
    if (cl < 1 || cl > 64 || (cl & (cl - 1)) != 0) return RFP4_ERR_UNSUPPORTED;
  }
  if (f.gemv_splits < 0 || f.gemv_splits > 4) return RFP4_ERR_UNSUPPORTED;
  if (f.gemv_split_combine != 0 && f.gemv_split_combine != 1) return RFP4_ERR_UNSUPPORTED;
  if (f.gemm_plan < RFP4_GEMM_PLAN_AUTO || f.gemm_plan > RFP4_GEMM_PLAN_NOSPLIT) return RFP4_ERR_UNSUPPORTED;
  *out = f;
  return RFP4_OK;
}

}  // namespace

extern "C" {

size_t rfp4_block_bytes(int layout) {
  return layout_ok(layout) ? static_cast<size_t>(rfp4::block_bytes(layout)) : 0;
}

int64_t rfp4_row_bytes(int layout, int64_t k) {
  if (!layout_ok(layout) || k < 32 || k > kMaxDim || (k % 32) != 0) return -1;
  return (k / 32) * rfp4::block_bytes(layout);
}

const char* rfp4_status_string(int status) {
  switch (status) {
    case RFP4_OK: return "ok";
    case RFP4_ERR_NULL: return "a required pointer is NULL";
    case RFP4_ERR_SHAPE: return "shape out of range (n, m, k, batch or a leading dimension)";
    case RFP4_ERR_UNSUPPORTED: return "unsupported layout, dtype or alignment";
    case RFP4_ERR_NONFINITE_SCALE: return "non-finite scale byte (low seven bits all ones)";
    case RFP4_ERR_HIP: return "HIP runtime error at launch";
    case RFP4_ERR_SCRATCH:
      return "the forced GEMM plan needs more partial-sum memory than the allocation-free entry point's "
             "static scratch array holds";
    default: return "unknown status";
  }
}

rfp4_status rfp4_validate(const uint8_t* w_host, int layout, int64_t n, int64_t k,
                          int64_t* first_bad_block) {
  if (first_bad_block) *first_bad_block = -1;
  if (!layout_ok(layout)) return RFP4_ERR_UNSUPPORTED;
  if (n < 1 || n > kMaxDim || k < 32 || k > kMaxDim || (k % 32) != 0) return RFP4_ERR_SHAPE;
  if (w_host == nullptr) return RFP4_ERR_NULL;
  const int bb = rfp4::block_bytes(layout);
  const int nscale = bb - 16;
  const int64_t blocks = n * (k / 32);
  const uint8_t* p = w_host + 16;  // first scale byte of block 0
  for (int64_t b = 0; b < blocks; ++b, p += bb) {
    for (int s = 0; s < nscale; ++s) {
      if ((p[s] & 0x7F) == 0x7F) {
        if (first_bad_block) *first_bad_block = b;
        return RFP4_ERR_NONFINITE_SCALE;
      }
    }
  }
  return RFP4_OK;
}

rfp4_status rfp4_dequant(const void* w, int layout, int64_t n, int64_t k, float* out,
                         int64_t ldo, void* stream) {
  rfp4_status st = check_weights(w, layout, n, k);
  if (st != RFP4_OK) return st;
  if (ldo < k || ldo > (int64_t(1) << 40) / n) return RFP4_ERR_SHAPE;
  if (out == nullptr) return RFP4_ERR_NULL;
  if (!aligned16(out) || (ldo % 4) != 0) return RFP4_ERR_UNSUPPORTED;
  return from_hip(rfp4::launch_dequant(static_cast<const uint8_t*>(w), layout, n, k, out, ldo,
                                       static_cast<hipStream_t>(stream)));
}

rfp4_status rfp4_gemv_multi_ex(int count, const void* const* w, const int64_t* n, int layout,
                               int64_t k, const void* x, int xdtype, int64_t batch, int64_t ldx,
                               float* const* y, const int64_t* ldy, const rfp4_force* force,
                               void* stream) {
  rfp4::Force f;
  if (check_force(force, &f) != RFP4_OK) return RFP4_ERR_UNSUPPORTED;
  if (count < 1 || count > RFP4_MAX_GEMV_PARTS) return RFP4_ERR_SHAPE;
  if (w == nullptr || n == nullptr || y == nullptr || ldy == nullptr) return RFP4_ERR_NULL;
  rfp4::GemvPart parts[rfp4::kMaxGemvParts];
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) {
    const rfp4_status st = check_weights(w[i], layout, n[i], k);
    if (st != RFP4_OK) return st;
    if (ldy[i] < n[i] || ldy[i] > kMaxDim) return RFP4_ERR_SHAPE;
    if (y[i] == nullptr) return RFP4_ERR_NULL;
    if (!aligned4(y[i])) return RFP4_ERR_UNSUPPORTED;
    rows += n[i];
    parts[i] = rfp4::GemvPart{static_cast<const uint8_t*>(w[i]), n[i], y[i], ldy[i]};
  }
  if (rows > kMaxDim) return RFP4_ERR_SHAPE;
  if (xdtype != RFP4_F16 && xdtype != RFP4_BF16) return RFP4_ERR_UNSUPPORTED;
  if (batch < 1 || batch > 8) return RFP4_ERR_SHAPE;
  if (ldx < k || ldx > kMaxDim) return RFP4_ERR_SHAPE;
  if (x == nullptr) return RFP4_ERR_NULL;
  if (!aligned4(x) || (ldx % 2) != 0) return RFP4_ERR_UNSUPPORTED;
  return from_hip(rfp4::launch_gemv(parts, count, layout, k, x, xdtype, static_cast<int>(batch),
                                    ldx, f, static_cast<hipStream_t>(stream)));
}

rfp4_status rfp4_gemv_multi(int count, const void* const* w, const int64_t* n, int layout,
                            int64_t k, const void* x, int xdtype, int64_t batch, int64_t ldx,
                            float* const* y, const int64_t* ldy, void* stream) {
  return rfp4_gemv_multi_ex(count, w, n, layout, k, x, xdtype, batch, ldx, y, ldy, nullptr, stream);
}

rfp4_status rfp4_gemv(const void* w, int layout, int64_t n, int64_t k, const void* x,
                      int xdtype, int64_t batch, int64_t ldx, float* y, int64_t ldy,
                      void* stream) {
  return rfp4_gemv_multi_ex(1, &w, &n, layout, k, x, xdtype, batch, ldx, &y, &ldy, nullptr, stream);
}

rfp4_status rfp4_dequant_bf16(const void* w, int layout, int64_t n, int64_t k, uint16_t* out,
                              int64_t ldo, void* stream) {
  rfp4_status st = check_weights(w, layout, n, k);
  if (st != RFP4_OK) return st;
  if (ldo < k || ldo > kMaxElems / n) return RFP4_ERR_SHAPE;
  if (out == nullptr) return RFP4_ERR_NULL;
  if (!aligned16(out) || (ldo % 8) != 0) return RFP4_ERR_UNSUPPORTED;
  return from_hip(rfp4::launch_dequant_bf16(static_cast<const uint8_t*>(w), layout, n, k, out, ldo,
                                            static_cast<hipStream_t>(stream)));
}

namespace {
// Shared checks of the GEMM entry points (weights, A, C).
rfp4_status check_gemm(const void* w, int layout, int64_t n, int64_t k, const void* a, int64_t m,
                       int64_t lda, const void* c, int64_t ldc) {
  rfp4_status st = check_weights(w, layout, n, k);
  if (st != RFP4_OK) return st;
  if (m < 1 || m > kMaxDim) return RFP4_ERR_SHAPE;
  if (lda < k || ldc < n || lda > kMaxDim || ldc > kMaxDim) return RFP4_ERR_SHAPE;
  if (lda > kMaxElems / m || ldc > kMaxElems / m) return RFP4_ERR_SHAPE;
  if (a == nullptr || c == nullptr) return RFP4_ERR_NULL;
  if (!aligned4(a) || !aligned4(c) || (lda % 2) != 0) return RFP4_ERR_UNSUPPORTED;
  return RFP4_OK;
}
}  // namespace

rfp4_status rfp4_gemm_dequant(const void* w, int layout, int64_t n, int64_t k, const void* a,
                              int64_t m, int64_t lda, void* c, int64_t ldc, uint16_t* wbuf,
                              int64_t ldw, void* stream) {
  rfp4_status st = check_gemm(w, layout, n, k, a, m, lda, c, ldc);
  if (st != RFP4_OK) return st;
  if (ldw < k || ldw > kMaxElems / n) return RFP4_ERR_SHAPE;
  if (wbuf == nullptr) return RFP4_ERR_NULL;
  if (!aligned16(wbuf) || (ldw % 8) != 0) return RFP4_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = from_hip(rfp4::launch_dequant_bf16(static_cast<const uint8_t*>(w), layout, n, k, wbuf, ldw, s));
  if (st != RFP4_OK) return st;
  return static_cast<rfp4_status>(rfp4::dense_gemm_bf16(wbuf, n, k, ldw, static_cast<const uint16_t*>(a),
                                                        m, lda, static_cast<uint16_t*>(c), ldc, s));
}

rfp4_status rfp4_gemm_ex(const void* w, int layout, int64_t n, int64_t k, const void* a,
                         int64_t m, int64_t lda, void* c, int64_t ldc, const rfp4_force* force,
                         void* stream) {
  rfp4::Force f;
  if (check_force(force, &f) != RFP4_OK) return RFP4_ERR_UNSUPPORTED;
  rfp4_status st = check_gemm(w, layout, n, k, a, m, lda, c, ldc);
  if (st != RFP4_OK) return st;
  return from_hip(rfp4::launch_gemm(static_cast<const uint8_t*>(w), layout, n, k,
                                    static_cast<const uint16_t*>(a), m, lda,
                                    static_cast<uint16_t*>(c), ldc, f,
                                    static_cast<hipStream_t>(stream)));
}

rfp4_status rfp4_gemm_noalloc(const void* w, int layout, int64_t n, int64_t k, const void* a,
                              int64_t m, int64_t lda, void* c, int64_t ldc, const rfp4_force* force,
                              void* stream) {
  rfp4::Force f;
  if (check_force(force, &f) != RFP4_OK) return RFP4_ERR_UNSUPPORTED;
  rfp4_status st = check_gemm(w, layout, n, k, a, m, lda, c, ldc);
  if (st != RFP4_OK) return st;
  if (rfp4::gemm_noalloc_plan_bytes(n, k, m, f) > static_cast<double>(RFP4_GEMM_SCRATCH_BYTES))
    return RFP4_ERR_SCRATCH;
  return from_hip(rfp4::launch_gemm_noalloc(static_cast<const uint8_t*>(w), layout, n, k,
                                            static_cast<const uint16_t*>(a), m, lda,
                                            static_cast<uint16_t*>(c), ldc, f,
                                            static_cast<hipStream_t>(stream)));
}

rfp4_status rfp4_gemm(const void* w, int layout, int64_t n, int64_t k, const void* a,
                      int64_t m, int64_t lda, void* c, int64_t ldc, void* stream) {
  return rfp4_gemm_ex(w, layout, n, k, a, m, lda, c, ldc, nullptr, stream);
}

rfp4_status rfp4_quantize(const void* src, int src_dtype, int64_t n, int64_t k, int64_t lds,
                          int layout, void* w_out, void* stream) {
  if (!layout_ok(layout)) return RFP4_ERR_UNSUPPORTED;
  if (src_dtype != RFP4_F32 && src_dtype != RFP4_BF16 && src_dtype != RFP4_F16)
    return RFP4_ERR_UNSUPPORTED;
  if (n < 1 || n > kMaxDim || k < 32 || k > kMaxDim || (k % 32) != 0) return RFP4_ERR_SHAPE;
  if (lds < k || lds > kMaxElems / n) return RFP4_ERR_SHAPE;
  if (src == nullptr || w_out == nullptr) return RFP4_ERR_NULL;
  const int64_t esize = src_dtype == RFP4_F32 ? 4 : 2;
  if (!aligned16(src) || !aligned16(w_out) || (lds * esize) % 16 != 0) return RFP4_ERR_UNSUPPORTED;
  return from_hip(rfp4::launch_quantize(src, src_dtype, n, k, lds, layout,
                                        static_cast<uint8_t*>(w_out),
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
