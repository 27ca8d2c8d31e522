// One fused decode step: the step's TensorScatter of the new K and V rows, its
// static-cache bias build and the split-KV attention in one launch (mobius
// skill "attention-optimization", "In-place KV for ONNX Attention via
// TensorScatter (static cache)": the cache write, the bias and the attention
// of a step; mobius issue #366, "Mobius-side deliverable": the bias rules).
// Results: those of kv_scatter_and_bias followed by attn_bias_gqa_fwd with that
// bias, bit for bit. The kernel is the decode kernel of decode_kernel.h in its
// step form (the in-kernel rules mask the scores, the side outputs are
// written by workgroups that never wait for one another); instantiated here,
// apart from the attention-only forms, so the two compile in parallel.
#include "decode_kernel.h"

namespace abgqa {

template <int D, int DV, int NR, int NW>
static void launch_step_nw(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.n_split));
  hipLaunchKernelGGL((attn_decode_kernel<D, DV, NR, NW, true, uint16_t, true>), grid, dim3(NW * 64), 0,
                     stream, p);
}

template <int D, int DV, int NR>
static hipError_t launch_step_d(const AttnParams& p, hipStream_t stream) {
  constexpr int NW = decode_waves<D, DV, NR>();
  // the instantiation the attention-only launch picks for the same shape
  if constexpr (decode_has_eight<D, DV, NR>()) {
    if (decode_use_eight(p)) launch_step_nw<D, DV, NR, 8>(p, stream);
    else launch_step_nw<D, DV, NR, NW>(p, stream);
  } else {
    launch_step_nw<D, DV, NR, NW>(p, stream);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) set_launch_detail("decode step kernel launch");
  return e;
}

template <int D, int DV>
static hipError_t launch_step_nr(const AttnParams& p, hipStream_t stream) {
  const int R = p.S_q * p.G;
  if (R <= 1) return launch_step_d<D, DV, 1>(p, stream);
  if (R <= 2) return launch_step_d<D, DV, 2>(p, stream);
  if (R <= 4) return launch_step_d<D, DV, 4>(p, stream);
  if (R <= 8) return launch_step_d<D, DV, 8>(p, stream);
  return launch_step_d<D, DV, 16>(p, stream);
}

hipError_t launch_decode_step(const AttnParams& p, hipStream_t stream) {
  if (p.bias != nullptr || p.S_new < 0 || p.S_new > 16) return hipErrorInvalidValue;
  if (p.D == p.Dv) {
    switch (p.D) {
      case 64: return launch_step_nr<64, 64>(p, stream);
      case 128: return launch_step_nr<128, 128>(p, stream);
      case 256: return launch_step_nr<256, 256>(p, stream);
      case 512: return launch_step_nr<512, 512>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.D == 256 && p.Dv == 512) return launch_step_nr<256, 512>(p, stream);
  if (p.D == 512 && p.Dv == 256) return launch_step_nr<512, 256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace abgqa
