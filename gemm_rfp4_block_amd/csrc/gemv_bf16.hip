// Fused dequant + GEMV kernels for bf16 activations (see gemv_impl.h).

#include "gemv_mfma.h"

namespace rfp4 {

hipError_t launch_gemv_bf16(const GemvPart* parts, int count, int layout, int nb, const uint16_t* x,
                          int batch, int64_t ldx, const Force& force, hipStream_t stream) {
  if (use_mfma(parts, count, nb, batch, force))
    return launch_gemv_mfma_xt<kBF16>(parts, count, layout, nb, x, batch, ldx, force, stream);
  return launch_gemv_xt<kBF16>(parts, count, layout, nb, x, batch, ldx, force, stream);
}

}  // namespace rfp4
