// Fused dequant + GEMV kernels for f16 activations (see gemv_impl.h).

#include "gemv_mfma.h"
#include "gemv_tall.h"

namespace rfp4 {

hipError_t launch_gemv_f16(const GemvPart* parts, int count, int layout, int nb, const uint16_t* x,
                          int batch, int64_t ldx, const Force& force, hipStream_t stream) {
  if (use_mfma(parts, count, nb, batch, force))
    return launch_gemv_mfma_xt<kF16>(parts, count, layout, nb, x, batch, ldx, force, stream);
  if (gemv_tall_fits(parts, count, layout, nb, batch, force)) return launch_gemv_tall(parts, count, nb, x, stream);
  return launch_gemv_xt<kF16>(parts, count, layout, nb, x, batch, ldx, force, stream);
}

}  // namespace rfp4
