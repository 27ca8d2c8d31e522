// The static-cache mask predicate, evaluated on the device by the bias builder
// and by the in-kernel-rules variant of the attention kernels.
//
// mobius issue #366, "Mobius-side deliverable": key validity slot < nonpad,
// combined with the causal, sliding-window, block-overlay and padding rules,
// keyed on the absolute query position q = q_start[b] + s.
//   valid    j < nonpad (clamped to [0, max_seq]) and kind[j] >= 0 (not a pad)
//   causal   j <= q
//   window   q - j < W  (keys [q-W+1, q]; W <= 0: no window) - mobius skill
//            "attention-optimization", "GQA sliding window via local_window_size"
//   block    kind[q] > 0 and kind[j] == kind[q] (bidirectional image block)
//   allowed  valid and ((causal and window) or block)
// Default q_start = max(nonpad - S_q, 0): the bottom-right offset of an external
// cache (onnxruntime skill "cuda-attention-kernel-patterns", section 11). All
// position arithmetic is signed (same skill, section 12).
#pragma once

#include "common.h"

namespace abgqa {

struct RowRule {
  int64_t np;      // valid slots, clamped to [0, max_seq]
  int64_t q;       // absolute query position
  int64_t window;  // <= 0: none
  int32_t kind_q;  // kind of the query slot (0 outside the cache)

  __device__ __forceinline__ bool allowed(int64_t j, int32_t kind_j) const {
    const bool valid = (j < np) && (kind_j >= 0);
    const bool causal = j <= q;
    const bool in_window = (window <= 0) || (q - j < window);
    const bool block = (kind_q > 0) && (kind_j == kind_q);
    return valid && ((causal && in_window) || block);
  }
};

__device__ __forceinline__ int64_t default_q_start(int64_t np, int64_t S_q) {
  const int64_t qs = np - S_q;
  return qs < 0 ? 0 : qs;
}

__device__ __forceinline__ RowRule make_row_rule(const int64_t* nonpad, const int64_t* q_start,
                                                 const int32_t* slot_kind, int64_t b, int64_t s,
                                                 int64_t S_q, int64_t max_seq, int64_t window) {
  RowRule r;
  r.np = clamp_nonpad(nonpad[b], max_seq);
  const int64_t qs = q_start ? q_start[b] : default_q_start(r.np, S_q);
  r.q = qs + s;
  r.window = window;
  r.kind_q = (slot_kind && r.q >= 0 && r.q < max_seq) ? slot_kind[b * max_seq + r.q] : 0;
  return r;
}

}  // namespace abgqa
