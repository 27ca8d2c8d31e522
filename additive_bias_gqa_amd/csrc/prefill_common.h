// Shared pieces of the two bf16 prefill paths (attn_prefill.hip: register-
// staged K/V tiles, any alignment; attn_prefill_dma.hip: direct-to-LDS tile
// pipeline for 16-byte-aligned rows): matrix-core and LDS helpers, the
// swizzled tile layout and the live-tile list.
#pragma once

#include "common.h"
#include "kernels.h"
#include "mask_rules.h"

namespace abgqa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kTileKeys = 32;
constexpr float kRescaleThreshold = 8.f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// gfx950 transposing LDS read: within each group of 16 lanes, lane i receives
// element (i % 4) of the 4-element (8-byte) row addressed by lane 4*k + i/4 of
// the same group, for k = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const __bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// XOR pattern applied to the 16-byte chunk index of tile row r (the LDS has
// 64 banks of 4 bytes: a 16-byte read serves 16 lanes per cycle, a transposing
// 8-byte read 32 lanes). For rows of at least 16 chunks (D >= 128) it is
// 4 bits wide and
//   - over any 16 consecutive rows a permutation of 0..15: 16 lanes reading
//     one chunk of 16 rows hit 16 distinct 16-byte bank groups;
//   - over rows 8a..8a+7 it maps the chunk pair {2m, 2m+1} of each row to 16
//     distinct chunks (16-row transposing reads: 8 rows x 32 bytes);
//   - over rows 4a..4a+3 it maps the chunk quad {4m..4m+3} of each row to 16
//     distinct chunks (32-row transposing reads: 4 rows x 64 bytes).
// Rows of 8 chunks (D = 64) take the 3-bit analogue. A plain r & 7 leaves
// two- to four-way conflicts on the transposing reads.
template <int D>
__device__ __forceinline__ int swz_bits(int r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  else return ((r & 3) << 1) | ((r >> 2) & 1);
}
template <int D>
constexpr int swz_width() { return D >= 128 ? 4 : 3; }

// element offset of 16-byte chunk c of row r in a swizzled [rows][D] tile
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return r * D + 8 * (c ^ swz_bits<D>(r));
}

__host__ __device__ inline int num_tiles(int n) { return (n + kTileKeys - 1) / kTileKeys; }

template <typename BiasT>
__device__ __forceinline__ bool live_bits(BiasT v);
template <>
__device__ __forceinline__ bool live_bits<uint16_t>(uint16_t v) { return v != 0xFF80; }
template <>
__device__ __forceinline__ bool live_bits<uint32_t>(uint32_t v) { return v != 0xFF800000u; }

template <typename BiasT>
__device__ __forceinline__ float bias_f32(BiasT v);
template <>
__device__ __forceinline__ float bias_f32<uint16_t>(uint16_t v) { return bf16_bits_to_f32(v); }
template <>
__device__ __forceinline__ float bias_f32<uint32_t>(uint32_t v) { return __uint_as_float(v); }

}  // namespace

// The live 32-key tiles of one workgroup's query rows [s0, s_end): tiles below
// nonpad that hold an allowed entry for one of the rows. Bias variant: scanned
// from the bias rows. Rules variant: the causal/window range of the rows plus
// every tile holding a slot of an image block that one of the rows belongs to
// (up to 4 distinct blocks; more makes every tile live). Skipping a dead tile
// is exact: its keys contribute exactly zero. Returns the count; the tile
// indices are in s_list[0 .. count).
// map_row (bias variant): this workgroup's words of a live-tile map built by
// tilemap_kernel for the same rows - copied instead of scanning the bias.
template <int NT, bool kRules, typename BiasT>
__device__ __forceinline__ int build_live_list(const AttnParams& p, int64_t b, int np, int s0, int s_end, int n_kt,
                               uint32_t* s_bits, uint16_t* s_list, int n_words, int32_t* s_ids,
                               int* s_nids_p, int* s_nlive_p,
                               const uint32_t* map_row = nullptr, uint32_t map_pre = 0u) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int T = p.T;
  int& s_nids = *s_nids_p;
  int& s_nlive = *s_nlive_p;
  for (int i = tid; i < n_words; i += NT) s_bits[i] = 0u;
  if (tid == 0) { s_nids = 0; s_nlive = 0; }
  if (tid < 4) s_ids[tid] = -1;  // never a block id: a racing reader cannot match it
  __syncthreads();
  if (!kRules && map_row) {
    // map_pre: word tid of map_row, already loaded by the caller (n_words <= NT)
    if (tid < n_words) s_bits[tid] = map_pre;
  } else if constexpr (!kRules) {
    // NB 16-byte loads per thread in flight at once, unconditional (index
    // clamped to the last vector, the copies discarded), so the scan costs one
    // memory round trip per batch rather than one per load
    constexpr int EPV = 16 / sizeof(BiasT);
    constexpr int NB = 16;
    const int nvec = (np + EPV - 1) / EPV;
    const BiasT* bb = (const BiasT*)p.bias + (b * p.S_q) * (int64_t)T;
    const int total = (s_end - s0) * nvec;
    if ((T % EPV) == 0) {
      for (int base = tid; base < total; base += NB * NT) {
        u32x4 raw[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int idx = min(base + u * NT, total - 1);
          const int sr = idx / nvec;
          raw[u] = ld_global<u32x4>(bb + (int64_t)(s0 + sr) * T + (idx - sr * nvec) * EPV);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int idx = base + u * NT;
          const int j0 = (idx % nvec) * EPV;
          BiasT vals[EPV];
          *reinterpret_cast<u32x4*>(vals) = raw[u];
          bool any = false;
#pragma unroll
          for (int e = 0; e < EPV; ++e) any |= (j0 + e < np) && live_bits<BiasT>(vals[e]);
          if (any && idx < total) {
            const int t = j0 / kTileKeys;   // EPV divides the tile size
            atomicOr(&s_bits[t >> 5], 1u << (t & 31));
          }
        }
      }
    } else {
      for (int idx = tid; idx < total; idx += NT) {
        const int sr = idx / nvec;
        const int j0 = (idx - sr * nvec) * EPV;
        const BiasT* row = bb + (int64_t)(s0 + sr) * T;
        bool any = false;
        for (int e = 0; e < EPV; ++e) any |= (j0 + e < np) && live_bits<BiasT>(row[j0 + e]);
        if (any) {
          const int t = j0 / kTileKeys;
          atomicOr(&s_bits[t >> 5], 1u << (t & 31));
        }
      }
    }
  } else {
    // causal + window: the rows' key intervals lie in [a, z] (q is consecutive
    // over the rows); a circular cache: in the slots of positions
    // [max(q_first - W + 1, oldest held), min(q_last, L - 1)], one interval or,
    // wrapping round the slots, two ([a, z] and [a2, z2])
    int a = 0, z = -1, a2 = 0, z2 = -1;
    if (p.circular) {
      if (s_end > s0) {
        const RowRule r0 = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s0, p.S_q, T, p.window, true);
        const int64_t L = p.nonpad[b] < 0 ? 0 : p.nonpad[b];
        const int64_t oldest = L > T ? L - T : 0;
        const int64_t q_last = r0.q + (s_end - 1 - s0);
        int64_t plo = p.window > 0 ? r0.q - p.window + 1 : 0;
        if (plo < oldest) plo = oldest;
        const int64_t phi = q_last < L - 1 ? q_last : L - 1;
        if (plo <= phi) {
          if (phi - plo + 1 >= T) {
            z = np - 1;
          } else {
            a = (int)(plo % T);
            z = (int)(phi % T);
            if (a > z) {   // wraps: [a, T - 1] and [0, z]
              a2 = 0;
              z2 = z;
              z = T - 1;
            }
          }
        }
      }
    } else if (s_end > s0) {
      const RowRule r0 = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s0, p.S_q, T, p.window, p.circular);
      const int64_t q_last = r0.q + (s_end - 1 - s0);
      int64_t a64 = (p.window > 0) ? r0.q - p.window + 1 : 0;
      if (a64 < 0) a64 = 0;
      const int64_t z64 = q_last < (int64_t)np - 1 ? q_last : (int64_t)np - 1;
      a = (int)(a64 < T ? a64 : T);
      z = (int)(z64 < -1 ? -1 : z64);
    }
    if (!p.slot_kind) {
      // every slot is text: the interval(s) alone
      if (a <= z)
        for (int t = a / kTileKeys + tid; t <= z / kTileKeys; t += NT) atomicOr(&s_bits[t >> 5], 1u << (t & 31));
      if (a2 <= z2)
        for (int t = a2 / kTileKeys + tid; t <= z2 / kTileKeys; t += NT) atomicOr(&s_bits[t >> 5], 1u << (t & 31));
    } else {
      // the rows' image-block kinds (up to 4 distinct; more: any block key counts)
      for (int s = s0 + tid; s < s_end; s += NT) {
        const RowRule rr = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window, p.circular);
        if (rr.kind_q > 0) {
          bool seen = false;
          for (int i = 0; i < 4; ++i) seen |= (i < s_nids) && (s_ids[i] == rr.kind_q);
          if (!seen) {
            const int slot = atomicAdd(&s_nids, 1);
            if (slot < 4) s_ids[slot] = rr.kind_q;
          }
        }
      }
      __syncthreads();
      const int nids = s_nids;
      // a tile is live if it holds a key that is no pad inside [a, z] or
      // [a2, z2], or a
      // key of one of the rows' blocks (a superset of the tiles some row
      // allows a key of; pad-only tiles drop out). Lanes 0-31 and 32-63 of a
      // wavefront read one tile each (NT is a multiple of 64), NB kinds per
      // thread in flight.
      const int32_t* kr = p.slot_kind + b * T;
      constexpr int NB = 8;
      for (int base0 = w * 64; base0 < np; base0 += NB * NT) {   // uniform over the wavefront
        const int base = base0 + lane;
        int32_t kv[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) kv[u] = kr[min(base + u * NT, np - 1)];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int j = base + u * NT;
          bool hit = (kv[u] >= 0) && (((j >= a) && (j <= z)) || ((j >= a2) && (j <= z2)));
          if (nids > 4) {
            hit |= kv[u] > 0;
          } else {
            for (int i = 0; i < nids; ++i) hit |= (kv[u] == s_ids[i]);
          }
          const uint64_t m = __ballot(hit && j < np);
          if (lane == 0 && m != 0) {
            const int t0 = (j - lane) / kTileKeys;   // the tile of lane 0
            if (m & 0xffffffffull) atomicOr(&s_bits[t0 >> 5], 1u << (t0 & 31));
            if (m >> 32) atomicOr(&s_bits[(t0 + 1) >> 5], 1u << ((t0 + 1) & 31));
          }
        }
      }
    }
  }
  __syncthreads();
  // compact the bitmap into a list (wavefront 0, 64 tiles per step)
  if (w == 0) {
    int base = 0;
    for (int t0 = 0; t0 < n_kt; t0 += 64) {
      const int t = t0 + lane;
      const bool live = (t < n_kt) && ((s_bits[t >> 5] >> (t & 31)) & 1u);
      const uint64_t mask = __ballot(live);
      const int pos = __popcll(mask & ((1ull << lane) - 1ull));
      if (live) s_list[base + pos] = (uint16_t)t;
      base += __popcll(mask);
    }
    if (lane == 0) s_nlive = base;
  }
  __syncthreads();
  return s_nlive;
}

}  // namespace abgqa
