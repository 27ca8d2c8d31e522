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
//
// Circular (window-sized) cache of capacity C = max_seq (reading of mobius
// skill "attention-optimization", "GQA sliding window via local_window_size",
// which names the circular cache as the way to bound a sliding layer's memory):
// nonpad carries L, the count of tokens written so far (absolute, may exceed
// C); the token of position p sits in slot p mod C, so slot j holds the newest
// position p < L with p = j (mod C) and is valid iff j < min(L, C). The rules
// above apply to that position; the query's kind is that of slot q mod C while
// position q is held (max(L - C, 0) <= q < L), else 0. The positions allowed by
// causal and window form one interval of at most C positions, so one or two
// slot intervals.
#pragma once

#include "common.h"

namespace abgqa {

struct RowRule {
  int64_t np = 0;      // valid slots, clamped to [0, max_seq]
  int64_t q = 0;       // absolute query position
  int64_t window = 0;  // <= 0: none
  int32_t kind_q = 0;  // kind of the query slot (0 outside the cache)
  // The same predicate in 32-bit form (max_seq < 2^30): causal-and-window is
  // the key interval [lo, hi], found once per row in 64-bit arithmetic (empty
  // when hi < lo), and a block key matches blk (-1, which no valid key has,
  // when the query slot starts no block). A default rule allows nothing.
  int32_t np32 = 0, lo = 0, hi = -1, blk = -1;
  // a second key interval: the wrapped part of a circular cache's interval
  // (empty for a static cache)
  int32_t lo2 = 0, hi2 = -1;

  __device__ __forceinline__ bool allowed(int j, int32_t kind_j) const {
    return (j < np32) & (kind_j >= 0) &
           (((j >= lo) & (j <= hi)) | ((j >= lo2) & (j <= hi2)) | (kind_j == blk));
  }
};

__device__ __forceinline__ int64_t default_q_start(int64_t np, int64_t S_q) {
  const int64_t qs = np - S_q;
  return qs < 0 ? 0 : qs;
}

__device__ __forceinline__ RowRule make_row_rule_circular(int64_t np_raw, bool has_qs,
                                                          int64_t qs_raw,
                                                          const int32_t* slot_kind, int64_t b,
                                                          int64_t s, int64_t S_q, int64_t C,
                                                          int64_t window) {
  RowRule r;
  const int64_t L = np_raw < 0 ? 0 : np_raw;
  r.np = L < C ? L : C;
  const int64_t qs = has_qs ? qs_raw : default_q_start(L, S_q);
  r.q = qs + s;
  r.window = window;
  const int64_t oldest = L > C ? L - C : 0;   // oldest position still held
  r.kind_q = (slot_kind && r.q >= oldest && r.q < L) ? slot_kind[b * C + r.q % C] : 0;
  // positions [plo, phi] allowed by causal and window among those held: at
  // most C of them, so slot (plo mod C) onwards, wrapping round once at most
  int64_t plo = window > 0 ? r.q - window + 1 : 0;
  if (plo < oldest) plo = oldest;
  const int64_t phi = r.q < L - 1 ? r.q : L - 1;
  r.np32 = (int32_t)r.np;
  r.blk = r.kind_q > 0 ? r.kind_q : -1;
  if (plo <= phi) {
    const int64_t a = plo % C, len = phi - plo + 1;
    r.lo = (int32_t)a;
    if (a + len <= C) {
      r.hi = (int32_t)(a + len - 1);
    } else {
      r.hi = (int32_t)(C - 1);
      r.lo2 = 0;
      r.hi2 = (int32_t)(a + len - 1 - C);
    }
  }
  return r;
}

// The rule of row (b, s) from nonpad[b] and q_start[b] already loaded (has_qs
// false: the default q_start); the one load left is the query slot's kind.
__device__ __forceinline__ RowRule make_row_rule_from(int64_t np_raw, bool has_qs, int64_t qs_raw,
                                                      const int32_t* slot_kind, int64_t b,
                                                      int64_t s, int64_t S_q, int64_t max_seq,
                                                      int64_t window, bool circular) {
  if (circular)
    return make_row_rule_circular(np_raw, has_qs, qs_raw, slot_kind, b, s, S_q, max_seq, window);
  RowRule r;
  r.np = clamp_nonpad(np_raw, max_seq);
  const int64_t qs = has_qs ? qs_raw : default_q_start(r.np, S_q);
  r.q = qs + s;
  r.window = window;
  r.kind_q = (slot_kind && r.q >= 0 && r.q < max_seq) ? slot_kind[b * max_seq + r.q] : 0;
  // keys j in [0, np) with j <= q and (no window or j >= q - W + 1)
  const int64_t lo = window > 0 ? r.q - window + 1 : 0;
  const int64_t hi = r.q < r.np - 1 ? r.q : r.np - 1;
  r.np32 = (int32_t)r.np;
  r.lo = (int32_t)(lo < 0 ? 0 : (lo > max_seq ? max_seq : lo));
  r.hi = (int32_t)(hi < -1 ? -1 : hi);
  r.blk = r.kind_q > 0 ? r.kind_q : -1;
  return r;
}

__device__ __forceinline__ RowRule make_row_rule(const int64_t* nonpad, const int64_t* q_start,
                                                 const int32_t* slot_kind, int64_t b, int64_t s,
                                                 int64_t S_q, int64_t max_seq, int64_t window,
                                                 bool circular = false) {
  return make_row_rule_from(nonpad[b], q_start != nullptr, q_start ? q_start[b] : 0, slot_kind, b,
                            s, S_q, max_seq, window, circular);
}

}  // namespace abgqa
