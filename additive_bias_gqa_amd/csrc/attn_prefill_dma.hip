// Dispatch of the direct-to-LDS prefill kernel (prefill_dma.h): which rows per
// wavefront and wavefronts per workgroup serve a head size, and when the path
// applies. Instantiations whose accumulators live in the ordinary vector
// registers are compiled here; the D = 512 kernel with 32-row wavefronts
// (accumulators in the accumulation registers) in attn_prefill_dma_wide.hip.
#include "prefill_dma.h"

namespace abgqa {

namespace {

// Rows per wavefront x wavefronts per workgroup for a shape. D = 512: 4
// wavefronts of 32 rows (Q^T in registers, O^T in the accumulation registers):
// each K/V tile fetched once for 128 rows, each LDS read feeding a 32-row MFMA.
// D = 256: 8 wavefronts of 16 rows, as 4 row groups x 2 key halves that take
// alternate tiles and merge at the end: 64 rows per workgroup like 4
// wavefronts, but two wavefronts per SIMD, each hiding the other's LDS and
// softmax latency (a prefill chunk rarely has the rows for two 16-row
// wavefronts per SIMD otherwise). D = 128: 4 wavefronts of 16 rows keep all
// four SIMDs of a CU busy with one workgroup per CU. D = 64 (a tile too small
// to split four ways): 32-row wavefronts, 4 of them when that still gives a
// workgroup per CU.
// the (D, DV) pairs with a V head size of their own that the kernel is built
// for (D = 256 beside DV = 512, and the reverse)
bool dma_dv_pair(int D, int Dv) { return (D == 256 && Dv == 512) || (D == 512 && Dv == 256); }

// Rows per workgroup of those pairs: 4 wavefronts of 32 rows (O^T in the
// accumulation registers) when that grid has a workgroup for every CU, else 4
// wavefronts of 16 rows (O^T in the ordinary registers, twice the
// workgroups). Vision-chunk shape (B 2, 8 KV heads, 512 tokens, G 2) with
// DV = 512: 63 us against 78; long-prefill shape with DV = 256 (1024
// workgroups of 32-row wavefronts): 298 us against 403.
int dv_rows(int64_t B, int64_t Hkv, int64_t S_q, int64_t G) {
  const int64_t wg32 = B * Hkv * ((S_q * G + 127) / 128);
  return wg32 >= 256 ? 128 : 64;
}

// query rows per workgroup of the D = DV kernels (see launch_dma_d)
int dma_rows(int D, int64_t B, int64_t Hkv, int64_t S_q, int64_t G) {
  if (D >= 512) return 128;
  if (D >= 128) return 64;
  const int64_t wg4 = B * Hkv * ((S_q * G + 127) / 128);
  return wg4 >= 256 ? 128 : 64;
}

template <int D>
hipError_t launch_dma_d(const AttnParams& p, hipStream_t stream) {
  if constexpr (D >= 512) {
    return launch_attn_prefill_dma_qreg(p, 4, stream);
  } else if constexpr (D == 256) {
    return launch_dma_v<D, 16, 8, true, 2>(p, stream);
  } else if constexpr (D == 128) {
    return launch_dma_v<D, 16, 4>(p, stream);
  } else {
    if (dma_rows(D, p.B, p.Hkv, p.S_q, p.G) == 128) return launch_dma_v<D, 32, 4>(p, stream);
    return launch_dma_v<D, 32, 2>(p, stream);
  }
}

}  // namespace

// The direct-to-LDS path needs 16-byte-aligned global chunks for every fetch:
// bias rows (max_seq * bias element size) and slot-kind rows (max_seq * 4) must
// be multiples of 16 bytes, and the live list must fit next to the stages: at
// kDmaMaxSeq slots it takes 2048 * 2 bytes of tile numbers and 64 map words
// (4.3 KiB of the 6 KiB the stages leave; every configuration has at least 128
// threads to load the 64 words). Its
// bias stage is sized for grouped heads (G >= 2: at most RW*NW/2 tokens per
// workgroup); one head per KV head takes the register-staged kernels.
bool prefill_dma_supported(const AttnParams& p) {
  if (p.D != 64 && p.D != 128 && p.D != 256 && p.D != 512) return false;
  if (p.Dv != p.D && !dma_dv_pair(p.D, p.Dv)) return false;
  if (p.G < 2) return false;   // the bias stage holds the rows of G >= 2 heads per token
  if (p.T > kDmaMaxSeq) return false;
  if (p.bias != nullptr) {
    if ((p.T % (p.bias_is_bf16 ? 8 : 4)) != 0) return false;
  } else if (p.slot_kind != nullptr) {
    if ((p.T % 4) != 0) return false;
  }
  return p.T >= 8;
}

// The live-tile map of the shape's configuration: one bit per (batch row,
// query tile, key tile). Shapes that take another path simply leave the
// scratch unused.
size_t prefill_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q, int64_t max_seq,
                               int64_t D, int64_t D_v) {
  if (D != 64 && D != 128 && D != 256 && D != 512) return 0;
  if (D_v != D && !dma_dv_pair((int)D, (int)D_v)) return 0;
  const int64_t G = Hq / Hkv;
  if (G < 2 || G > 64 || max_seq > kDmaMaxSeq) return 0;
  const int64_t rows = D_v != D ? dv_rows(B, Hkv, S_q, G) : dma_rows((int)D, B, Hkv, S_q, G);
  const int64_t mq = rows / G;
  const int64_t n_qt = (S_q + mq - 1) / mq;
  const int64_t n_words = (num_tiles((int)max_seq) + 31) / 32;
  return (size_t)(B * n_qt * n_words) * sizeof(uint32_t);
}

hipError_t launch_attn_prefill_dma(const AttnParams& p, hipStream_t stream) {
  // a V head size of its own
  if (p.Dv != p.D) {
    if (dv_rows(p.B, p.Hkv, p.S_q, p.G) == 64) {
      if (p.D == 256) return launch_dma_v<256, 16, 4, true, 1, 512>(p, stream);
      return launch_dma_v<512, 16, 4, true, 1, 256>(p, stream);
    }
    return launch_attn_prefill_dma_qreg(p, 4, stream);
  }
  switch (p.D) {
    case 64: return launch_dma_d<64>(p, stream);
    case 128: return launch_dma_d<128>(p, stream);
    case 256: return launch_dma_d<256>(p, stream);
    case 512: return launch_dma_d<512>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace abgqa
