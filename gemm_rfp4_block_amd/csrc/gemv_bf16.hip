// Fused dequant + GEMV kernels for bf16 activations (see gemv_impl.h).

#include "gemv_mfma.h"

namespace rfp4 {

hipError_t launch_gemv_bf16(const GemvPart* parts, int count, int layout, int nb, const uint16_t* x,
                          int batch, int64_t ldx, hipStream_t stream) {
  if (use_mfma(parts, count, nb, batch)) return launch_gemv_mfma_xt<kBF16>(parts, count, layout, nb, x, batch, ldx, stream);
  return launch_gemv_xt<kBF16>(parts, count, layout, nb, x, batch, ldx, stream);
}

}  // namespace rfp4
