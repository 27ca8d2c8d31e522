// bf16 split-KV decode attention: the host side (split count, workspace size,
// launch of the attention-only instantiations). The kernel and what it
// computes: decode_kernel.h.
#include <stdlib.h>

#include "decode_kernel.h"

namespace abgqa {

int decode_num_splits(int64_t B, int64_t Hkv, int64_t max_seq) {
  // ABGQA_DECODE_SPLITS (1..256) overrides the heuristic: rows of very uneven
  // live length over a long cache can gain from more splits than one per CU.
  // Read at every call, so the workspace size query and the call agree as long
  // as the variable does not change between them (a call whose workspace is too
  // small for its split count is refused).
  const char* v = getenv("ABGQA_DECODE_SPLITS");
  const int forced = v ? atoi(v) : 0;
  if (forced > 0) return forced > 256 ? 256 : forced;
  // The grid runs in rounds of 256 workgroups (one per CU): a round that is
  // only partly filled leaves CUs idle while the rest run, and the longest
  // workgroup of a round sets its end. Splits let the balancing pass (section
  // 1b of the kernel) even out rows of different live length, but each adds a
  // workgroup's fixed costs (range, merge, record). So: among the split counts
  // that keep the grid within two rounds, the one whose rounds are fullest;
  // ties go to fewer splits. One split once B * Hkv fills two rounds by itself.
  // Measured (decode over 8192 slots, head 512, lengths U{1024..8192}): B * Hkv
  // 48 -> 5 splits 105.6 us (6: 146.7), 96 -> 5 202.7 us (3: 271), 160 -> 3
  // 299.6 us (2: 391); sliding window 1024 over 4096 slots, head 256: 136 -> 3
  // 38.5 us (2: 45.1), 200 -> 1 42.1 us (2: 52.1).
  const int64_t P = B * Hkv;
  int64_t cap = (max_seq + 63) / 64;   // at least 64 slots per split
  if (cap > 64) cap = 64;
  if (cap < 1) cap = 1;
  int64_t best = 1, best_rounds = (P + 255) / 256;
  for (int64_t n = 2; n <= cap; ++n) {
    const int64_t rounds = (P * n + 255) / 256;
    if (rounds > 2) break;
    if (n * best_rounds > best * rounds) {   // fuller rounds: n / rounds larger
      best = n;
      best_rounds = rounds;
    }
  }
  return (int)best;
}

// workspace: the arrival counts, then one partial record per (kv head, rank),
// rank < B * n_split
size_t decode_workspace_bytes(int64_t B, int64_t Hkv, int64_t S_q, int64_t G, int64_t Dv,
                              int64_t max_seq) {
  const int64_t NR = round_up_rows(S_q * G);
  const int64_t n_split = decode_num_splits(B, Hkv, max_seq);
  return kWsCounterBytes + (size_t)B * Hkv * n_split * part_floats(NR, Dv) * sizeof(float);
}

template <int D, int DV, int NR, int NW>
static void launch_decode_nw(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.Hkv * p.n_split));
  if (p.bias == nullptr)
    hipLaunchKernelGGL((attn_decode_kernel<D, DV, NR, NW, true, uint16_t>), grid, dim3(NW * 64), 0, stream, p);
  else if (p.bias_is_bf16)
    hipLaunchKernelGGL((attn_decode_kernel<D, DV, NR, NW, false, uint16_t>), grid, dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_decode_kernel<D, DV, NR, NW, false, uint32_t>), grid, dim3(NW * 64), 0, stream, p);
}

template <int D, int DV, int NR>
static hipError_t launch_decode_d(const AttnParams& p, hipStream_t stream) {
  constexpr int NW = decode_waves<D, DV, NR>();
  if constexpr (decode_has_eight<D, DV, NR>()) {
    if (decode_use_eight(p)) launch_decode_nw<D, DV, NR, 8>(p, stream);
    else launch_decode_nw<D, DV, NR, NW>(p, stream);
  } else {
    launch_decode_nw<D, DV, NR, NW>(p, stream);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) set_launch_detail("decode kernel launch");
  return e;
}

template <int D, int DV>
static hipError_t launch_decode_nr(const AttnParams& p, hipStream_t stream) {
  const int R = p.S_q * p.G;
  if (R <= 1) return launch_decode_d<D, DV, 1>(p, stream);
  if (R <= 2) return launch_decode_d<D, DV, 2>(p, stream);
  if (R <= 4) return launch_decode_d<D, DV, 4>(p, stream);
  if (R <= 8) return launch_decode_d<D, DV, 8>(p, stream);
  return launch_decode_d<D, DV, 16>(p, stream);
}

// Head sizes the split-KV kernel is built for: every D with DV = D, and the
// pairs of the 256 / 512 heads of sliding and full-attention layers (a
// KV-shared layer reading the V of a layer with the other head size).
bool decode_supports(int D, int Dv) {
  if (D == Dv) return D == 64 || D == 128 || D == 256 || D == 512;
  return (D == 256 && Dv == 512) || (D == 512 && Dv == 256);
}

hipError_t launch_attn_decode(const AttnParams& p, hipStream_t stream) {
  if (p.D == p.Dv) {
    switch (p.D) {
      case 64: return launch_decode_nr<64, 64>(p, stream);
      case 128: return launch_decode_nr<128, 128>(p, stream);
      case 256: return launch_decode_nr<256, 256>(p, stream);
      case 512: return launch_decode_nr<512, 512>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.D == 256 && p.Dv == 512) return launch_decode_nr<256, 512>(p, stream);
  if (p.D == 512 && p.Dv == 256) return launch_decode_nr<512, 256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace abgqa
