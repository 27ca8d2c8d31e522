// Dispatch of the direct-to-LDS prefill kernel (prefill_dma.h): which rows per
// wavefront and wavefronts per workgroup serve a head size, and when the path
// applies. Instantiations whose accumulators live in the ordinary vector
// registers are compiled here; the D = 512 kernel with 32-row wavefronts
// (accumulators in the accumulation registers) in attn_prefill_dma_wide.hip.
#include "prefill_dma.h"

namespace abgqa {

namespace {

// ABGQA_PREFILL_CFG (tuning): "32x2", "32x4", "16x4", "16x8" picks rows per
// wavefront x wavefronts per workgroup ("32x2r", "32x4r": Q^T in registers);
// otherwise the default below.
static int prefill_cfg() {
  static const int v = [] {
    const char* e = getenv("ABGQA_PREFILL_CFG");
    if (!e) return 0;
    if (!strcmp(e, "32x2")) return 1;
    if (!strcmp(e, "32x4")) return 2;
    if (!strcmp(e, "16x4")) return 3;
    if (!strcmp(e, "16x8")) return 4;
    if (!strcmp(e, "32x2r")) return 5;
    if (!strcmp(e, "32x4r")) return 6;
    return 0;
  }();
  return v;
}

template <int D>
hipError_t launch_dma_d(const AttnParams& p, hipStream_t stream) {
  const int cfg = prefill_cfg();
  if constexpr (D >= 512) {
    if (cfg == 4) return launch_dma_v<D, 16, 8>(p, stream);
    if (cfg == 3) return launch_dma_v<D, 16, 4>(p, stream);
    // 4 wavefronts of 32 rows (Q^T in registers, O^T in the accumulation
    // registers): each K/V tile fetched once for 128 rows, each LDS read
    // feeding a 32-row MFMA
    return launch_attn_prefill_dma_qreg(p, 4, stream);
  } else {
    if constexpr (D == 256) {
      if (cfg == 5) return launch_attn_prefill_dma_qreg(p, 2, stream);
      if (cfg == 6) return launch_attn_prefill_dma_qreg(p, 4, stream);
    }
    if (cfg == 1) return launch_dma_v<D, 32, 2>(p, stream);
    if (cfg == 2) return launch_dma_v<D, 32, 4>(p, stream);
    if constexpr (D >= 128) {   // a tile must split evenly over the wavefronts
      if (cfg == 3) return launch_dma_v<D, 16, 4>(p, stream);
      if (cfg == 4) return launch_dma_v<D, 16, 8>(p, stream);
    }
    // D >= 128: 4 wavefronts of 16 rows keep all four SIMDs of a CU busy with
    // one workgroup per CU (64 rows; the LDS holds one workgroup's stages).
    // D = 64 (a tile too small to split four ways): 32-row wavefronts.
    if constexpr (D >= 128) return launch_dma_v<D, 16, 4>(p, stream);
    const int64_t wg4 = (int64_t)p.B * p.Hkv * ((p.S_q * (int64_t)p.G + 127) / 128);
    if (wg4 >= 256) return launch_dma_v<D, 32, 4>(p, stream);
    return launch_dma_v<D, 32, 2>(p, stream);
  }
}

}  // namespace

// The direct-to-LDS path needs 16-byte-aligned global chunks for every fetch:
// bias rows (max_seq * bias element size) and slot-kind rows (max_seq * 4) must
// be multiples of 16 bytes, and the live list must fit next to the stages. Its
// bias stage is sized for grouped heads (G >= 2: at most RW*NW/2 tokens per
// workgroup); one head per KV head takes the register-staged kernels.
bool prefill_dma_supported(const AttnParams& p) {
  if (p.D != 64 && p.D != 128 && p.D != 256 && p.D != 512) return false;
  if (p.G < 2) return false;   // the bias stage holds the rows of G >= 2 heads per token
  if (p.T > 32768) return false;
  if (p.bias != nullptr) {
    if ((p.T % (p.bias_is_bf16 ? 8 : 4)) != 0) return false;
  } else if (p.slot_kind != nullptr) {
    if ((p.T % 4) != 0) return false;
  }
  return p.T >= 8;
}

hipError_t launch_attn_prefill_dma(const AttnParams& p, hipStream_t stream) {
  switch (p.D) {
    case 64: return launch_dma_d<64>(p, stream);
    case 128: return launch_dma_d<128>(p, stream);
    case 256: return launch_dma_d<256>(p, stream);
    case 512: return launch_dma_d<512>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace abgqa
