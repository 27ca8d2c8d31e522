// Device bodies of the per-step preparation work, shared by the separate
// entry points (scatter.hip: TensorScatter; bias.hip: bias build) and by the
// fused one (prepare.hip: both K and V scatters and the bias in one launch).
// Each body is a grid-stride loop over its own work items, run by `nblk`
// workgroups of 256 threads numbered `blk`.
#pragma once

#include "common.h"
#include "mask_rules.h"

namespace abgqa {

// TensorScatter (mobius skill "attention-optimization", "In-place KV for ONNX
// Attention via TensorScatter (static cache)"): update row (b, h, t) lands in
// cache slot write_indices[b] + t; slots outside [0, max_seq) are dropped. A
// circular cache (mask_rules.h) takes position write_indices[b] + t in slot
// (position) mod max_seq instead, negative positions dropped. One thread moves
// 16 bytes of a row (of each of the two caches when cache2 is given: K and V
// rows of one head size, same write indices); a workgroup covers
// 256 / vec_per_row rows per step. Every load of a row (the update chunks and
// write_indices[b]) is issued before any is used, so a row costs one memory
// round trip before its stores.
__device__ __forceinline__ void scatter_rows(u32x4* __restrict__ cache,
                                             const u32x4* __restrict__ update,
                                             u32x4* __restrict__ cache2,
                                             const u32x4* __restrict__ update2,
                                             const int64_t* __restrict__ write_indices, int H,
                                             int max_seq, int S_new, int vec_per_row,
                                             int64_t n_rows, int64_t blk, int64_t nblk,
                                             bool circular) {
  const int rows_per_iter = 256 / vec_per_row;
  const int sub = threadIdx.x / vec_per_row;
  const int c = threadIdx.x % vec_per_row;
  if (sub >= rows_per_iter) return;
  const bool two = cache2 != nullptr;
  for (int64_t row = blk * rows_per_iter + sub; row < n_rows; row += nblk * rows_per_iter) {
    int64_t bh, b;
    int t;
    if (n_rows <= 0x7fffffff) {   // 32-bit divisions when the indices fit
      const uint32_t bh32 = (uint32_t)row / (uint32_t)S_new;
      t = (int)((uint32_t)row - bh32 * (uint32_t)S_new);
      bh = bh32;
      b = bh32 / (uint32_t)H;
    } else {
      bh = row / S_new;
      t = (int)(row - bh * S_new);
      b = bh / H;
    }
    const int64_t src = row * vec_per_row + c;
    const u32x4 u = update[src];
    const u32x4 u2 = (two ? update2 : update)[src];
    int64_t slot = (write_indices ? write_indices[b] : 0) + t;
    if (slot < 0) continue;                     // dropped
    if (circular) slot %= max_seq;
    else if (slot >= max_seq) continue;         // dropped (no wrap-around)
    const int64_t dst = (bh * max_seq + slot) * vec_per_row + c;
    cache[dst] = u;
    if (two) cache2[dst] = u2;
  }
}

// bits of +0.0 / -inf in the bias element type
template <typename T> struct MaskBits;
template <> struct MaskBits<uint16_t> {
  static constexpr uint16_t kZero = 0x0000, kNegInf = 0xFF80;
};
template <> struct MaskBits<uint32_t> {
  static constexpr uint32_t kZero = 0x00000000u, kNegInf = 0xFF800000u;
};

// Static-cache bias (mobius issue #366, "Mobius-side deliverable"; rule in
// mask_rules.h). One thread writes 8 consecutive keys of one (b, s) row; `vec`
// (max_seq % 8 == 0) selects 16-byte kind loads and bias stores.
template <typename T>
__device__ __forceinline__ void bias_chunks(T* __restrict__ bias, const int64_t* __restrict__ nonpad,
                                            const int64_t* __restrict__ q_start,
                                            const int32_t* __restrict__ slot_kind, int S_q,
                                            int max_seq, int64_t window, int chunks_per_row,
                                            int64_t n_chunks, bool vec, int64_t blk, int64_t nblk,
                                            bool circular) {
  for (int64_t idx = blk * 256 + threadIdx.x; idx < n_chunks; idx += nblk * 256) {
    int64_t row, b;
    int j0, s;
    if (n_chunks <= 0x7fffffff) {   // 32-bit divisions when the indices fit
      const uint32_t r32 = (uint32_t)idx / (uint32_t)chunks_per_row;
      const uint32_t b32 = r32 / (uint32_t)S_q;
      j0 = (int)((uint32_t)idx - r32 * (uint32_t)chunks_per_row) * 8;
      s = (int)(r32 - b32 * (uint32_t)S_q);
      row = r32;
      b = b32;
    } else {
      row = idx / chunks_per_row;
      j0 = (int)(idx - row * chunks_per_row) * 8;
      b = row / S_q;
      s = (int)(row - b * S_q);
    }
    const int32_t* kind_row = slot_kind ? slot_kind + b * max_seq : nullptr;
    // Every load that does not need the rule goes out first (the chunk's slot
    // kinds beside nonpad[b] and q_start[b]), so a chunk waits for two memory
    // round trips: those loads, then the query slot's kind.
    // (q_start is read without a branch: from nonpad when absent, unused then.)
    const int64_t np_raw = nonpad[b];
    const int64_t qs_raw = (q_start ? q_start : nonpad)[b];
    int4 k0 = make_int4(0, 0, 0, 0), k1 = make_int4(0, 0, 0, 0);
    if (vec && kind_row) {
      k0 = ld_global<int4>(kind_row + j0);
      k1 = ld_global<int4>(kind_row + j0 + 4);
    }
    const RowRule rule = make_row_rule_from(np_raw, q_start != nullptr, qs_raw, slot_kind, b, s, S_q,
                                            max_seq, window, circular);
    T* out = bias + row * max_seq + j0;
    if (vec) {
      const int32_t kinds[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      T v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = rule.allowed(j0 + e, kinds[e]) ? MaskBits<T>::kZero : MaskBits<T>::kNegInf;
      if constexpr (sizeof(T) == 2) {
        u32x4 w;
        w.x = v[0] | ((uint32_t)v[1] << 16);
        w.y = v[2] | ((uint32_t)v[3] << 16);
        w.z = v[4] | ((uint32_t)v[5] << 16);
        w.w = v[6] | ((uint32_t)v[7] << 16);
        *reinterpret_cast<u32x4*>(out) = w;
      } else {
        *reinterpret_cast<u32x4*>(out) = u32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<u32x4*>(out + 4) = u32x4{v[4], v[5], v[6], v[7]};
      }
    } else {
      for (int e = 0; e < 8 && j0 + e < max_seq; ++e) {
        const int32_t kj = kind_row ? kind_row[j0 + e] : 0;
        out[e] = rule.allowed(j0 + e, kj) ? MaskBits<T>::kZero : MaskBits<T>::kNegInf;
      }
    }
  }
}

}  // namespace abgqa
