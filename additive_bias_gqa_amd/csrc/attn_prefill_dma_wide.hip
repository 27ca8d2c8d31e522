// The direct-to-LDS prefill kernel (prefill_dma.h) with 32-row wavefronts and
// Q^T in registers, for D = 512 and for the pairs of a K head size and a V
// head size of its own (256 and 512 either way). Compiled without
// the ordinary-register form of the matrix-core accumulators: at D = 512 a
// lane holds 256 O^T accumulators beside 128 registers of Q^T fragments, so
// the accumulators take the accumulation registers and everything else the
// ordinary ones.
#include "prefill_dma.h"

namespace abgqa {

hipError_t launch_attn_prefill_dma_qreg(const AttnParams& p, int nw, hipStream_t stream) {
  if (p.D == 256 && p.Dv == 512 && nw == 4) return launch_dma_v<256, 32, 4, true, 1, 512>(p, stream);
  if (p.D == 512 && p.Dv == 256 && nw == 4) return launch_dma_v<512, 32, 4, true, 1, 256>(p, stream);
  if (p.Dv != p.D) return hipErrorInvalidValue;
  if (p.D == 512 && nw == 4) return launch_dma_v<512, 32, 4, true>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace abgqa
