// bf16 split-KV decode attention over the static cache (S_q * G <= 16 rows).
//
// What it computes: onnxruntime skill "cuda-attention-kernel-patterns",
// section 4 (scale * QK^T, + bias, softmax, times V), section 6 (a row with no
// allowed key, or nonpad = 0, writes zeros; masked keys removed by selection),
// section 11 (external cache: keys are the slots < nonpad_kv_seqlen); mobius
// issue #366 (the float bias carries causal/window/block/padding rules); query
// head h reads KV head h / G (onnxruntime PR #28242, CPU GQA excerpt).
//
// Why split-KV: decode is bound by memory bandwidth whatever the kernel
// (mobius skill "attention-optimization", "Flash Attention: when it actually
// helps"), and the decode edge of the grouped-query op comes from a dedicated
// single-token kernel (same skill, "In-place KV ... static cache"). So every
// KV byte is read once, by one of n_split workgroups per (batch, KV head), and
// every such read is shared by the G query heads of the group.
//
// Layout of the work
//   grid      B * Hkv * n_split workgroups of 4 wavefronts (8 for heads of
//             512 with up to 4 rows per lane group, and for heads of 256 with
//             up to 4 when the grid is one round); consecutive logical ids
//             (the splits of one (b, kv head)) share an XCD. n_split fills
//             whole rounds of 256 workgroups (decode_num_splits).
//   rows      r = s * G + g (query token s, head g of the group), R <= 16;
//             the 16 rows of the matrix-core tile are padded with zeros.
//   live      [lo, hi): the first and last key any row may attend, found from
//             the bias (or from the rules: the same keys, pads at the ends of
//             the causal/window interval excluded, so both forms split alike
//             and give the same bits); split i takes an even share of it.
//   block     16 keys per wavefront step (block i by one wavefront: i mod
//             NW, or unevenly between the two wavefronts of a SIMD, see
//             blk_wave):
//             S = Q K^T on the matrix cores (K read straight from HBM into the
//             B-operand registers, 16 bytes per lane, non-temporal like the V
//             loads: every K/V byte is read once), online softmax on the
//             S layout (lane = key, 4 rows per lane), then O += P V on the
//             vector ALU with V rows read coalesced (lane = 8 values of d).
//             The softmax weights cross layouts through a small LDS buffer.
//   merge     the wavefronts merge in LDS in a fixed order (bit-
//             reproducible); each workgroup writes its (m, l, O) partial to
//             the workspace and counts its arrival; the last of a row's
//             splits to arrive merges the row's partials:
//             m = max m_i, y = sum 2^(m_i - m) O_i / sum 2^(m_i - m) l_i.
//             The partials travel through agent-scope stores and loads,
//             which are coherent across the XCDs by themselves: no fence that
//             writes back or invalidates an L2 cache is needed (such fences,
//             once per workgroup, made an earlier form of this merge five
//             times slower than a separate combine kernel).
//
// Softmax runs in base 2 on x * log2(e). The running maximum is only raised
// when a new score exceeds it by more than 8 (a factor 256), so rescaling the
// accumulators is rare; weights stay <= 2^8 and the result is unchanged.
//
// The kernel template; its instantiations live in attn_decode.hip (attention
// only) and attn_decode_step.hip (the fused decode step).
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mask_rules.h"

namespace abgqa {

namespace {

constexpr float kRescaleThreshold = 8.f;

template <typename BiasT>
__device__ __forceinline__ bool bias_live_bits(BiasT v);
template <>
__device__ __forceinline__ bool bias_live_bits<uint16_t>(uint16_t v) { return v != 0xFF80; }
template <>
__device__ __forceinline__ bool bias_live_bits<uint32_t>(uint32_t v) { return v != 0xFF800000u; }

template <typename BiasT>
__device__ __forceinline__ float bias_value(BiasT v);
template <>
__device__ __forceinline__ float bias_value<uint16_t>(uint16_t v) { return bf16_bits_to_f32(v); }
template <>
__device__ __forceinline__ float bias_value<uint32_t>(uint32_t v) { return __uint_as_float(v); }

}  // namespace

static inline int64_t round_up_rows(int64_t R) {
  int64_t nr = 1;
  while (nr < R) nr *= 2;
  return nr;
}

// floats of one partial record: O[NR][D], then m[NR], l[NR], padded to 16 bytes
__host__ __device__ constexpr int64_t part_floats(int64_t NR, int64_t D) {
  return (NR * D + 2 * NR + 3) & ~(int64_t)3;
}

// Rows whose live ranges every split workgroup learns (several splits per row:
// then B * Hkv < 256 with the default split count)
constexpr int kMaxBalanceRows = 256;
// keys between the samples that estimate a row's live length (128: the
// split counts of a 16-row, 8192-key decode come out as an exact whole-split
// allocation would give them; 256 left the longest split 2.5% longer)
constexpr int kSampleStride = 128;

// Wavefronts per split workgroup: heads of 512 with up to 4 rows per lane
// group take 8 (two per SIMD, one block in flight each: more bytes in flight
// than 4 wavefronts with a prefetch buffer, and their registers hold the work
// without spilling); the rest take 4 with the prefetch buffer.
template <int D, int DV, int NR>
constexpr int decode_waves() {
  return (NR <= 4 && (D > DV ? D : DV) >= 512) ? 8 : 4;
}
// Heads of 256 with up to 4 rows per lane group also have an eight-wavefront
// form (two per SIMD, one block in flight each, blocks dealt as for head 512),
// launched when the grid is one round of at most 256 workgroups: the sliding
// decode step (B 8, Hkv 8, 4 splits) 20.45 -> 20.0 us with 2 rows per KV head,
// 23.3 -> 21.5 us with 4, its circular form 20.7 -> 20.0. Above 256
// workgroups the four-wavefront form stays, whose workgroups (up to 2 rows)
// can share a CU (B 12: 28.6 against 34.3 us with eight). Not for 8 rows (the
// eight-wavefront form spills) nor for heads of 128 (15.5 -> 15.7 us, slower).
template <int D, int DV, int NR>
constexpr bool decode_has_eight() {
  return (D > DV ? D : DV) == 256 && NR <= 4;
}
inline bool decode_use_eight(const AttnParams& p) {
  return (int64_t)p.B * p.Hkv * p.n_split <= 256;
}

// Agent-scope (whole-GPU) stores and loads: they complete at, and read from,
// the level every XCD shares, so a record written by a workgroup on one XCD is
// read back exactly by a workgroup on another, without writing back or
// invalidating any L2 cache.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at once (sc1: agent scope). There is no 16-byte scoped-store
// builtin, so this is asm, which the compiler does not count among the
// outstanding stores: the explicit s_waitcnt vmcnt(0) that follows the record
// stores waits for them.
__device__ __forceinline__ void st_agent4(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" :: "v"(p), "v"(v) : "memory");
}
// two floats in one agent-scope 8-byte load
__device__ __forceinline__ void ld_agent2(const float* p, float& x, float& y) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  x = __uint_as_float((uint32_t)u);
  y = __uint_as_float((uint32_t)(u >> 32));
}

// Wavefronts per SIMD the register allocation must allow. The head-256
// kernels with up to 2 rows and the smaller heads with up to 8 fit in 256
// registers without spilling, which lets two workgroups share a CU: a grid of
// more than 256 workgroups (several splits per row, or B * Hkv > 256) then
// runs at once instead of in two rounds (B 40, Hkv 8, sliding window 1024,
// head 256: 79.9 -> 76.4 us). Larger ones keep one wavefront per SIMD (the
// head-512 kernels already run two, at eight wavefronts per workgroup).
template <int D, int DV, int NR, int NW>
constexpr int decode_min_waves_per_simd() {
  constexpr int H = D > DV ? D : DV;
  return (NW == 4 && ((H <= 256 && NR <= 2) || (H <= 128 && NR <= 8))) ? 2 : 1;
}

// D: head size of Q and K; DV: of V and the output (they may differ)
template <int D, int DV, int NR, int NW, bool kRules, typename BiasT, bool kStep = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(decode_min_waves_per_simd<D, DV, NR, NW>())))
void attn_decode_kernel(AttnParams p) {
  static_assert(!kStep || kRules, "the fused step masks with the in-kernel rules");
  constexpr int kDecThreads = NW * 64;
  constexpr int kDecWaves = NW;
  constexpr int KSTEPS = D / 32;    // matrix-core k-steps over the head dim
  constexpr int LPR = DV / 8;       // lanes per V row (8 bf16 per lane)
  constexpr int KPI = 64 / LPR;     // V rows per wavefront load
  constexpr int NV = 16 / KPI;      // V loads per 16-key block
  constexpr int PART = (int)part_floats(NR, DV);
  constexpr int E = NR < 4 ? NR : 4;      // real rows per lane group (r = 4*grp + e)
  // the A operand (Q) in LDS only for D = 512 (its 64 registers per lane do
  // not fit beside the rest at two wavefronts per SIMD); below that in
  // registers, which keeps its reads off the LDS queue of every block
  constexpr bool kQinLds = D >= 512;

  __shared__ float s_p[kDecWaves][16][NR];  // softmax weights, key-major
  __shared__ float s_alpha[kDecWaves][NR];
  __shared__ float s_m[kDecWaves][NR];
  __shared__ float s_l[kDecWaves][NR];
  // wave merge: each wave's rescaled O in its own slot, summed in a fixed order
  // (one barrier), unless that needs more than 32 KiB: then accumulate wave by
  // wave into one buffer
  constexpr bool kParMerge = NW * NR * DV <= 8192;
  __shared__ float s_o[kParMerge ? NW * NR * DV : NR * DV];
  __shared__ __align__(16) __bf16 s_q[kQinLds ? NR * D : 8];  // Q rows (A operand)
  __shared__ int s_rlo[kDecWaves], s_rhi[kDecWaves];
  // rules variant: the 32-bit rule of each query token s < S_q of batch row b,
  // made once per workgroup (the lanes read it instead of loading nonpad,
  // q_start and the query slot's kind themselves)
  __shared__ int32_t s_rule[16][8];
  // several splits per row: live samples of every batch row
  __shared__ int s_cnt[kMaxBalanceRows];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int T = p.T, G = p.G, R = p.S_q * p.G;

  // ---- 0. which (kv head, batch row, split) ----------------------------------
  // Workgroups are numbered (kv head, rank), rank < B * n_split. With one split
  // per row the rank is the batch row. With several, rows of very different
  // live length would leave the workgroups of short rows idle while those of
  // the longest row run on, so every workgroup of a kv head first learns the
  // live key count of every batch row from samples (the same data
  // everywhere, hence the same answer) and the rows get splits in proportion
  // to it (section 1b). Until then b is the equal-split guess, which starts the Q
  // loads; a workgroup whose row changes loads Q again.
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int S = p.B * p.n_split;   // workgroups per kv head
  const int hk = wg / S;
  const int rank = wg % S;
  const bool multi = p.n_split > 1 && p.B <= kMaxBalanceRows;
  const int64_t b_guess = rank / p.n_split;
  int64_t b = b_guess;

  // ---- 0a. fused decode step: the loads of its two side outputs --------------
  // The launch also does the step's TensorScatter of K and V and its bias
  // build, and no workgroup waits for another: rank r < B of each kv head
  // writes batch row r's new K/V rows into the cache; the wavefront that
  // streams a slot this step writes stores that slot's update row itself
  // before its own loads of it (section 2b); the workgroups of a guessed batch
  // row (Hkv * n_split of them) share that row's bias chunks, so every chunk
  // of every row is written once. The attention masks with the in-kernel
  // rules, which give exactly the mask the bias holds. The loads go out here
  // (they retire before the range scan's, which the workgroup waits for
  // anyway); the stores go out later (sections 1a and 2b, side_stores).
  constexpr int KCH = D / 8, VCH = DV / 8;   // 16-byte chunks of a K / V row
  const bool st_writer = kStep && rank < p.B && p.S_new > 0;
  const int st_nch = kStep ? p.S_new * (KCH + VCH) : 0;   // chunks of a writer
  // chunk c of the writer: update row t = c / (KCH + VCH), of K below KCH
  auto st_src = [&](int c) -> const bf16x8* {
    const int t = c / (KCH + VCH), wc = c - t * (KCH + VCH);
    const int64_t row = ((int64_t)rank * p.Hkv + hk) * p.S_new + t;
    return wc < KCH ? (const bf16x8*)p.k_upd + row * KCH + wc
                    : (const bf16x8*)p.v_upd + row * VCH + (wc - KCH);
  };
  // TensorScatter of chunk c: position w + t, dropped when negative (or,
  // static cache, past the last slot); circular: slot = position mod T
  auto st_put = [&](int c, const bf16x8& v, int64_t w_own) {
    const int t = c / (KCH + VCH), wc = c - t * (KCH + VCH);
    int64_t pos = w_own + t;
    if (pos < 0 || (!p.circular && pos >= T)) return;
    if (p.circular) pos %= T;
    const int64_t row = ((int64_t)rank * p.Hkv + hk) * T + pos;
    bf16x8* dst = wc < KCH ? (bf16x8*)p.k + row * KCH + wc : (bf16x8*)p.v + row * VCH + (wc - KCH);
    *dst = v;
  };
  // eight bias values from an allow mask (bit e: key j0 + e allowed)
  auto put_bias8 = [&](int64_t off, uint32_t allow) {
    if (p.bias_out_bf16) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wv[e] = ((allow >> (2 * e)) & 1 ? 0u : 0xFF80u) | ((allow >> (2 * e + 1)) & 1 ? 0u : 0xFF800000u);
      *reinterpret_cast<u32x4*>((uint16_t*)p.bias_out + off) = u32x4{wv[0], wv[1], wv[2], wv[3]};
    } else {
      uint32_t wv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = (allow >> e) & 1 ? 0u : 0xFF800000u;
      uint32_t* o = (uint32_t*)p.bias_out + off;
      *reinterpret_cast<u32x4*>(o) = u32x4{wv[0], wv[1], wv[2], wv[3]};
      *reinterpret_cast<u32x4*>(o + 4) = u32x4{wv[4], wv[5], wv[6], wv[7]};
    }
  };
  bf16x8 st_val{};
  int64_t st_w_own = 0;
  int64_t st_wpos = 0;   // write position of the row this workgroup streams
  // update row 0 of the guessed batch row (its K then V chunks, chunk
  // lane + 64 i), for the wavefront that streams its slot (section 2b;
  // reloaded in section 1c when the assignment moves the workgroup to another
  // row)
  constexpr int UPL = (KCH + VCH + 63) / 64;
  bf16x8 st_row[UPL];
  auto upd_chunk = [&](int64_t bq, int t, int c) -> const bf16x8* {
    const int64_t row = (bq * p.Hkv + hk) * p.S_new + t;
    return c < KCH ? (const bf16x8*)p.k_upd + row * KCH + c
                   : (const bf16x8*)p.v_upd + row * VCH + (c - KCH);
  };
  if constexpr (kStep) {
    if (p.S_new > 0) {
#pragma unroll
      for (int i = 0; i < UPL; ++i)
        st_row[i] = ld_global<bf16x8>(upd_chunk(b_guess, 0, min(lane + 64 * i, KCH + VCH - 1)));
    }
    if (st_writer && tid < st_nch) st_val = ld_global<bf16x8>(st_src(tid));
    if (p.write_idx) {
      if (st_writer) st_w_own = p.write_idx[rank];
      st_wpos = p.write_idx[b_guess];
    }
  }
  // bias chunks (8 keys each) of the guessed row: workgroup wid of the row's
  // st_nw takes the contiguous chunks [wid * st_cpw, (wid + 1) * st_cpw) (whole
  // cache lines, written by one workgroup), chunk c0 + k * NT for thread tid
  const int st_cpr = (T + 7) / 8;
  const int st_nw = p.Hkv * p.n_split;
  const int st_all = kStep && p.bias_out ? p.S_q * st_cpr : 0;
  const int st_cpw = (st_all + st_nw - 1) / st_nw;
  const int st_wid = hk * p.n_split + rank % p.n_split;
  const int st_total = min(st_all, (st_wid + 1) * st_cpw);   // this workgroup's end
  const int st_c0 = st_wid * st_cpw + tid;
  const bool st_vec = (T % 8) == 0;
  int4 st_k0 = make_int4(0, 0, 0, 0), st_k1 = make_int4(0, 0, 0, 0);
  if constexpr (kStep) {
    if (st_c0 < st_total && st_vec && p.slot_kind) {
      const int32_t* kr = p.slot_kind + b_guess * T + (st_c0 % st_cpr) * 8;
      st_k0 = ld_global<int4>(kr);
      st_k1 = ld_global<int4>(kr + 4);
    }
  }

  // ---- 0b. Q rows (row r = s * G + g) into registers, to be parked in LDS ----
  // Issued before the range scan so that both memory round trips overlap; the
  // index is clamped (loads stay unconditional), the store is guarded.
  constexpr int QCH = kQinLds ? (NR * (D / 8) + kDecThreads - 1) / kDecThreads : 1;
  bf16x8 qtmp[QCH];
  auto load_q = [&](int64_t bq) {
    if constexpr (kQinLds) {
      const int nq = R * (D / 8);
#pragma unroll
      for (int i = 0; i < QCH; ++i) {
        const int c = min(tid + i * kDecThreads, nq - 1);
        const int r = c / (D / 8), dc = c % (D / 8);
        qtmp[i] = ld_global<bf16x8>((const __bf16*)p.q +
            (((bq * p.Hq + hk * G + r % G) * p.S_q + r / G) * (int64_t)D) + 8 * dc);
      }
    }
  };
  load_q(b);

  // ---- 1. live key ranges ----------------------------------------------------
  // (no memory fence before the scan: waiting here for the Q loads above would
  // put two memory round trips ahead of the K/V loads)
  if constexpr (!kParMerge)
    for (int i = tid; i < NR * DV; i += kDecThreads) s_o[i] = 0.f;
  // this row's exact range (bias variant): every key below nonpad whose bias
  // is not -inf, over the S_q rows, reduced into s_rlo / s_rhi per wavefront.
  // NB loads per thread in flight at once, unconditional (index clamped to the
  // last vector; the extra copies are discarded), so the scan costs one memory
  // round trip; the vector path reads whole rows (max_seq keys) and applies
  // j < nonpad afterwards, so its loads do not wait for nonpad first.
  auto scan_own = [&](int64_t bq) {
    int lo = INT32_MAX, hi = -1;
    if constexpr (!kRules) {
      const int npq = (int)clamp_nonpad(p.nonpad[bq], T);
      constexpr int EPV = 16 / sizeof(BiasT);  // elements per 16-byte load
      constexpr int NB = 4;
      const BiasT* bb = (const BiasT*)p.bias + bq * p.S_q * (int64_t)T;
      const bool vec_rows = (T % EPV) == 0;
      const int nvec = vec_rows ? T / EPV : (npq + EPV - 1) / EPV;
      const int total = p.S_q * nvec;
      if (vec_rows) {
        for (int base = tid; base < total; base += NB * kDecThreads) {
          u32x4 raw[NB];
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            const int idx = min(base + u * kDecThreads, total - 1);
            const int s = idx / nvec;
            raw[u] = ld_global<u32x4>(bb + (int64_t)s * T + (idx - s * nvec) * EPV);
          }
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            const int idx = base + u * kDecThreads;
            const int j0 = (idx % nvec) * EPV;
            BiasT vals[EPV];
            *reinterpret_cast<u32x4*>(vals) = raw[u];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
              const int j = j0 + e;
              if (idx < total && j < npq && bias_live_bits<BiasT>(vals[e])) {
                lo = min(lo, j);
                hi = max(hi, j);
              }
            }
          }
        }
      } else {
        for (int idx = tid; idx < total; idx += kDecThreads) {
          const int s = idx / nvec;
          const int j0 = (idx - s * nvec) * EPV;
          const BiasT* row = bb + (int64_t)s * T;
          for (int e = 0; e < EPV; ++e) {
            const int j = j0 + e;
            if (j < npq && bias_live_bits<BiasT>(row[j])) {
              lo = min(lo, j);
              hi = max(hi, j);
            }
          }
        }
      }
      lo = wave_min_i32(lo);
      hi = wave_max_i32(hi);
      if (lane == 0) { s_rlo[w] = lo; s_rhi[w] = hi; }
    }
  };
  // Live estimate of every batch row (several splits per row): the number of
  // sampled keys j = 128 i + 64 below nonpad that some query row of the batch
  // row allows - the bias entry not -inf, or the in-kernel rule, which gives
  // the same mask, so both variants balance alike. One load (or rule) per
  // sample: 64 per row of 8192 keys.
  auto make_rules = [&](int64_t bq) {
    if constexpr (kRules) {
      if (tid < p.S_q) {
        const RowRule rr = make_row_rule(p.nonpad, p.q_start, p.slot_kind, bq, tid, p.S_q, T, p.window, p.circular);
        // whether a pad slot ends one of the row's causal/window intervals:
        // then the interval is wider than the keys the row allows (the kinds
        // at the ends are loaded in the same round trip as the query slot's)
        int pad_end = 0;
        if (p.slot_kind) {
          const int32_t* kr = p.slot_kind + bq * T;
          if (rr.lo <= rr.hi) pad_end |= (kr[rr.lo] < 0) | (kr[rr.hi] < 0);
          if (rr.lo2 <= rr.hi2) pad_end |= (kr[rr.lo2] < 0) | (kr[rr.hi2] < 0);
        }
        int32_t* d = s_rule[tid];
        d[0] = rr.np32; d[1] = rr.lo; d[2] = rr.hi; d[3] = rr.blk;
        d[4] = rr.lo2; d[5] = rr.hi2; d[6] = rr.kind_q; d[7] = pad_end;
      }
    }
  };
  make_rules(b);
  if (multi) {
    for (int i = tid; i < p.B; i += kDecThreads) s_cnt[i] = 0;
    lds_barrier();
  }
  scan_own(b);
  if (multi) {
    const int ns = (T + kSampleStride - 1) / kSampleStride;
    for (int i = tid; i < p.B * ns; i += kDecThreads) {
      const int bb = i / ns;
      const int j = (i - bb * ns) * kSampleStride + kSampleStride / 2;
      bool live = false;
      if constexpr (kRules) {
        // nonpad, q_start and the sample's kind together, then the query
        // slots' kinds: two memory round trips
        const int64_t np_raw = p.nonpad[bb];
        const int64_t qs_raw = (p.q_start ? p.q_start : p.nonpad)[bb];
        const int32_t kj = p.slot_kind ? p.slot_kind[bb * (int64_t)T + min(j, T - 1)] : 0;
        if (j < (int)clamp_nonpad(np_raw, T)) {
          for (int s = 0; s < p.S_q; ++s) {
            const RowRule rr = make_row_rule_from(np_raw, p.q_start != nullptr, qs_raw, p.slot_kind,
                                                  bb, s, p.S_q, T, p.window, p.circular);
            live |= rr.allowed(j, kj);
          }
        }
      } else if (j < (int)clamp_nonpad(p.nonpad[bb], T)) {
        const BiasT* col = (const BiasT*)p.bias + (int64_t)bb * p.S_q * T + j;
        for (int s = 0; s < p.S_q; ++s) live |= bias_live_bits<BiasT>(col[(int64_t)s * T]);
      }
      if (live) atomicAdd(&s_cnt[bb], 1);
    }
  }
  __syncthreads();

  // ---- 1a. fused decode step: the side outputs ---------------------------------
  // Each thread's first writer chunk (st_val) and first bias chunk (its allow
  // mask, st_allow) are stored later (side_stores): stores issued now would sit
  // ahead of the first K/V loads in the memory counter the stream waits on. Further chunks (more than one per thread: long caches,
  // several query tokens or new tokens) are stored here.
  int st_allow = -1;
  if constexpr (kStep) {
    if (st_writer)
      for (int c = tid + kDecThreads; c < st_nch; c += kDecThreads) st_put(c, ld_global<bf16x8>(st_src(c)), st_w_own);
    // the bias (mobius issue #366, "Mobius-side deliverable"): +0 where the
    // guessed row's rule allows the key, -inf elsewhere; the rules are in s_rule
    for (int c = st_c0, k = 0; c < st_total; c += kDecThreads, ++k) {
      const int s = c / st_cpr, j0 = (c - s * st_cpr) * 8;
      RowRule rr;
      const int32_t* d = s_rule[s];
      rr.np32 = d[0]; rr.lo = d[1]; rr.hi = d[2]; rr.blk = d[3]; rr.lo2 = d[4]; rr.hi2 = d[5];
      const int32_t* kr = p.slot_kind ? p.slot_kind + b_guess * T : nullptr;
      const int64_t off = (b_guess * p.S_q + s) * (int64_t)T + j0;
      if (st_vec) {
        int4 k0 = st_k0, k1 = st_k1;
        if (k > 0 && kr) { k0 = ld_global<int4>(kr + j0); k1 = ld_global<int4>(kr + j0 + 4); }
        const int32_t kinds[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        uint32_t allow = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) allow |= rr.allowed(j0 + e, kinds[e]) ? (1u << e) : 0u;
        if (k == 0) st_allow = (int)allow;
        else put_bias8(off, allow);
      } else {
        for (int e = 0; e < 8 && j0 + e < T; ++e) {
          const bool ok = rr.allowed(j0 + e, kr ? kr[j0 + e] : 0);
          if (p.bias_out_bf16) ((uint16_t*)p.bias_out)[off + e] = ok ? 0u : 0xFF80u;
          else ((uint32_t*)p.bias_out)[off + e] = ok ? 0u : 0xFF800000u;
        }
      }
    }
  }
  // the deferred stores, issued once by every wavefront: right after its first
  // block's K/V loads (the wait for that block does not cover them, and they
  // are long complete when the next block is waited for) in the prefetching
  // stream, after the stream otherwise, or before a workgroup without work
  // returns
  auto side_stores = [&]() {
    if constexpr (kStep) {
      if (st_writer && tid < st_nch) st_put(tid, st_val, st_w_own);
      if (st_allow >= 0) {
        const int s = st_c0 / st_cpr, j0 = (st_c0 - s * st_cpr) * 8;
        put_bias8((b_guess * p.S_q + s) * (int64_t)T + j0, (uint32_t)st_allow);
      }
    }
  };

  // ---- 1b. splits per batch row ----------------------------------------------
  // Each wavefront computes the same assignment from the same LDS data. Rows
  // get nsp_b = max(1, ceil(c_b / X)) splits, c_b the live samples of row b,
  // X the smallest cap for which sum_b nsp_b <= B * n_split (a binary search),
  // when the busiest row has more than 1.25 times the mean; otherwise n_split
  // splits each. Ranks past sum_b nsp_b have no work.
  int split = rank % p.n_split, nsp = p.n_split, first = (int)b * p.n_split;
  if (multi) {
    int cnt4[4];
    int tot = 0, mx = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bb = lane + 64 * i;
      cnt4[i] = bb < p.B ? s_cnt[bb] : 0;
      tot += cnt4[i];
      mx = max(mx, cnt4[i]);
    }
    tot = wave_sum_i32(tot);
    mx = wave_max_i32(mx);
    if ((int64_t)mx * p.B * 4 > (int64_t)tot * 5) {
      int xl = 1, xh = mx;
      while (xl < xh) {
        const int xm = (xl + xh) >> 1;
        int need = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (lane + 64 * i < p.B) need += max(1, (cnt4[i] + xm - 1) / xm);
        need = wave_sum_i32(need);
        if (need <= S) xh = xm;
        else xl = xm + 1;
      }
      // batch row bb = lane + 64 i: prefix sums in row order, find this rank
      int carry = 0;
      int found = -1, f_first = 0, f_n = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bb = lane + 64 * i;
        const int n = bb < p.B ? max(1, (cnt4[i] + xl - 1) / xl) : 0;
        const int incl = wave_incl_sum_i32(n) + carry;
        const int fst = incl - n;
        if (n > 0 && rank >= fst && rank < fst + n) { found = bb; f_first = fst; f_n = n; }
        carry = __builtin_amdgcn_readlane(incl, 63);
      }
      const uint64_t hit = __ballot(found >= 0);
      if (hit == 0) {         // a rank past every row's splits: no work
        side_stores();
        return;
      }
      const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
      b = __builtin_amdgcn_readlane(found, src);
      first = __builtin_amdgcn_readlane(f_first, src);
      nsp = __builtin_amdgcn_readlane(f_n, src);
      split = rank - first;
    }
  }

  // ---- 1c. this row's live range [live_lo, live_hi) ---------------------------
  if constexpr (kRules) {
    // causal / window keys of every query row, then the image block of any row
    if (b != b_guess) {
      // the fused step's bias chunks (section 1a) read the guessed row's rules;
      // the new row's write position and update row 0 share the rules' memory
      // round trip
      if constexpr (kStep) {
        if (p.S_new > 0) {
          if (p.write_idx) st_wpos = p.write_idx[b];
#pragma unroll
          for (int i = 0; i < UPL; ++i)
            st_row[i] = ld_global<bf16x8>(upd_chunk(b, 0, min(lane + 64 * i, KCH + VCH - 1)));
        }
        __syncthreads();
      }
      make_rules(b);
    }
    __syncthreads();
    bool any_block = false, pad_end = false;
    for (int s = 0; s < p.S_q; ++s) {
      any_block |= s_rule[s][6] > 0;
      pad_end |= s_rule[s][7] != 0;
    }
    int lo = INT32_MAX, hi = -1;
    if (tid < p.S_q && !pad_end) {
      // the row's causal/window key interval(s) below nonpad (a circular
      // cache's may wrap round into a second one), exact at both ends
      const int32_t* d = s_rule[tid];
      if (d[1] <= d[2]) { lo = d[1]; hi = d[2]; }
      if (d[4] <= d[5]) { lo = min(lo, d[4]); hi = max(hi, d[5]); }
    }
    if (pad_end) {
      // a pad ends an interval: the first and last key that some row allows,
      // from the kinds of every valid slot (the bias variant's scan finds the
      // same two keys in the bias)
      const int32_t* kr = p.slot_kind + b * T;
      const int np = s_rule[0][0];
      for (int j = tid; j < np; j += kDecThreads) {
        const int32_t kj = kr[j];
        for (int s = 0; s < p.S_q; ++s) {
          const int32_t* d = s_rule[s];
          RowRule rr;
          rr.np32 = d[0]; rr.lo = d[1]; rr.hi = d[2]; rr.blk = d[3]; rr.lo2 = d[4]; rr.hi2 = d[5];
          if (rr.allowed(j, kj)) { lo = min(lo, j); hi = max(hi, j); break; }
        }
      }
    } else if (any_block) {
      const int32_t* kr = p.slot_kind + b * T;
      const int np = s_rule[0][0];   // valid slots of the row
      for (int j = tid; j < np; j += kDecThreads) {
        const int32_t kj = kr[j];
        if (kj <= 0) continue;
        for (int s = 0; s < p.S_q; ++s) {
          if (s_rule[s][6] == kj) { lo = min(lo, j); hi = max(hi, j); break; }
        }
      }
    }
    lo = wave_min_i32(lo);
    hi = wave_max_i32(hi);
    if (lane == 0) { s_rlo[w] = lo; s_rhi[w] = hi; }
    __syncthreads();
  } else if (b != b_guess) {
    // the row changed with the assignment: scan the new one
    scan_own(b);
    __syncthreads();
  }
  int live_lo = INT32_MAX, live_hi = 0;
#pragma unroll
  for (int ww = 0; ww < kDecWaves; ++ww) {
    live_lo = min(live_lo, s_rlo[ww]);
    live_hi = max(live_hi, s_rhi[ww] + 1);
  }
  if (live_hi <= live_lo) { live_lo = 0; live_hi = 0; }
  if constexpr (kQinLds) {
    if (b != b_guess) load_q(b);
#pragma unroll
    for (int i = 0; i < QCH; ++i) {
      const int c = tid + i * kDecThreads;
      if (c < R * (D / 8))
        *reinterpret_cast<bf16x8*>(&s_q[(c / (D / 8)) * D + 8 * (c % (D / 8))]) = qtmp[i];
    }
  }
  __syncthreads();
  const int live = live_hi - live_lo;
  const int per = ((live + nsp - 1) / nsp + 15) & ~15;
  const int my_lo = live_lo + split * per;
  const int my_hi = min(live_hi, my_lo + per);

  // ---- 2. per-lane row data -------------------------------------------------
  // lane layouts: Q as the A operand (row lane % 16, d-slots 32*i + 8*(lane/16),
  // loaded in section 2c); S with key lane % 16 and rows 4*(lane/16) + e
  const int qrow = lane & 15;
  const int kgrp = lane >> 4;
  // rows this lane holds in the S layout: r = 4 * kgrp + e
  int row_s[E];
  bool row_ok[E];
  RowRule rules[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int r = 4 * kgrp + e;
    row_ok[e] = r < R;
    row_s[e] = row_ok[e] ? r / G : 0;
    if constexpr (kRules) {
      const int32_t* d = s_rule[row_s[e]];
      rules[e].np32 = d[0]; rules[e].lo = d[1]; rules[e].hi = d[2]; rules[e].blk = d[3];
      rules[e].lo2 = d[4]; rules[e].hi2 = d[5];
    }
  }
  const float scale_log2 = p.scale * kLog2e;
  const bool cap_on = p.softcap > 0.f;
  const float cap2 = p.softcap * kLog2e, scale_over_cap = cap_on ? p.scale / p.softcap : 0.f;

  const __bf16* kbase = (const __bf16*)p.k + (b * p.Hkv + hk) * (int64_t)T * D;
  const __bf16* vbase = (const __bf16*)p.v + (b * p.Hkv + hk) * (int64_t)T * DV;
  const BiasT* biasb = kRules ? nullptr : (const BiasT*)p.bias + b * p.S_q * (int64_t)T;
  const int32_t* kindb = p.slot_kind ? p.slot_kind + b * T : nullptr;
  // the next block's K/V are loaded while this one is computed, except with
  // eight wavefronts (section 3)
  constexpr bool kPrefetch = NW == 4;
  // Which wavefront streams block i (keys my_lo + 16 i ...). One wavefront per
  // SIMD: block i goes to wavefront i % NW. Two per SIMD (NW = 8, waves w and
  // w + 4 share a SIMD, w launched first): the SIMD issues the older
  // wavefront's instructions first when both are ready, so with equal shares
  // the younger ones (4..7) stream about a third slower (measured on the
  // 16-row, 8192-slot, head-512 decode: 96 against 72 us) and run on alone
  // after the older ones finish, one block in flight per SIMD. So waves 0..3
  // take the first 11/16 of the blocks (block i to wave i % 4) and waves 4..7
  // the rest (block n_old + i to wave 4 + i % 4); shares of 8/16 to 14/16
  // measured, 11/16 fastest with the K/V loads non-temporal (12/16 before).
  // A fixed function of the split, so results stay bit-identical from run to
  // run.
  constexpr bool kTwoPerSimd = NW == 8;
  static_assert(!kTwoPerSimd || !kPrefetch, "two wavefronts per SIMD stream one block at a time");
  // sixteenths of the blocks for waves 0..3 (head 256: 12/16 fastest of 8,
  // 11 to 14)
  constexpr int kOldShare = (D > DV ? D : DV) >= 512 ? 11 : 12;
  const int n_blk = my_hi > my_lo ? (my_hi - my_lo + 15) >> 4 : 0;
  const int n_old = kTwoPerSimd ? (n_blk * kOldShare + 15) / 16 : n_blk;
  auto blk_wave = [&](int i) {
    if constexpr (kTwoPerSimd) return i < n_old ? (i & 3) : 4 + ((i - n_old) & 3);
    else return i % NW;
  };
  // the wavefront's own first block
  auto blk_first = [&](int i) {
    if constexpr (kTwoPerSimd) return i < n_old ? i < 4 : i - n_old < 4;
    else return i < NW;
  };
  // ---- 2b. fused decode step: the written slots this workgroup streams -------
  // Row b's update rows t in [st_tlo, st_thi) go to slots st_wb + t (mod T for
  // a circular cache). The wavefront that streams such a slot first stores the
  // slot's update row into the cache itself: its own loads of the slot follow
  // those stores in its program order, so they return the new row, whatever
  // the designated writer (which writes the same bytes) does meanwhile. No
  // other workgroup reads the slot (the splits' ranges are disjoint), and the
  // other wavefronts load it at most as a clamped index whose data is never
  // used. So the stream itself is the attention-only kernel's.
  // A slot in the wavefront's first block is stored before the stream; one in a
  // later block after the first block's loads (see side_stores), where the
  // stores do not sit ahead of loads the stream waits for next.
  int st_wb = 0, st_tlo = 0, st_thi = 0;
  if constexpr (kStep) {
    if (p.S_new > 0) {
      const int64_t wpos = st_wpos;
      if (p.circular) {
        st_wb = (int)(((wpos % T) + T) % T);
        st_tlo = (int)min<int64_t>(p.S_new, max<int64_t>(0, -wpos));
        st_thi = p.S_new;
      } else if (wpos < T && wpos + p.S_new > 0) {
        st_wb = (int)wpos;
        st_tlo = (int)max<int64_t>(0, -wpos);
        st_thi = (int)min<int64_t>(p.S_new, T - wpos);
      }
    }
  }
  // which: 0 = slots in this wavefront's first block, 1 = in its later blocks,
  // 2 = all of its slots
  auto reader_stores = [&](int which) {
    if constexpr (kStep) {
      for (int t = st_tlo; t < st_thi; ++t) {
        int j = st_wb + t;
        if (p.circular && j >= T) j -= T;
        if (j < my_lo || j >= my_hi || blk_wave((j - my_lo) >> 4) != w) continue;
        const bool first = blk_first((j - my_lo) >> 4);
        if ((which == 0 && !first) || (which == 1 && first)) continue;
        const int64_t slot = (b * p.Hkv + hk) * (int64_t)T + j;
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
          const int c = lane + 64 * i;
          if (c >= KCH + VCH) break;
          const bf16x8 v = t == 0 ? st_row[i] : ld_global<bf16x8>(upd_chunk(b, t, c));
          bf16x8* dst = c < KCH ? (bf16x8*)p.k + slot * KCH + c : (bf16x8*)p.v + slot * VCH + (c - KCH);
          *dst = v;
        }
      }
    }
  };
  reader_stores(kPrefetch ? 0 : 2);

  // ---- 2c. Q as the A operand (head sizes below 512: in registers) -----------
  // Issued only now: the memory counter retires in order, so a wait for any
  // earlier load (the step's write position, the update rows the reader stores
  // above hold) would otherwise also wait for these cold loads, a whole memory
  // round trip ahead of the first K/V loads. Unconditional (rows past R load
  // row 0 and take zeros), so no exec-masked branch hides their count.
  bf16x8 qa[kQinLds ? 1 : KSTEPS];
  if constexpr (!kQinLds) {
    const bool ok = qrow < R;
    const int s = ok ? qrow / G : 0, g = ok ? qrow % G : 0;
    const __bf16* qp = (const __bf16*)p.q +
        (((b * p.Hq + hk * G + g) * p.S_q + s) * (int64_t)D) + 8 * kgrp;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      const bf16x8 v = ld_global<bf16x8>(qp + 32 * i);
      qa[i] = ok ? v : bf16x8{};
    }
  }

  float m_run[E], l_run[E];
#pragma unroll
  for (int e = 0; e < E; ++e) { m_run[e] = -INFINITY; l_run[e] = 0.f; }
  float o[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[r][c] = 0.f;

  const int vkey = lane / LPR;       // key offset within a V load
  const int vd = 8 * (lane % LPR);   // first d of this lane in the PV layout

  // ---- 3. stream 16-key blocks (block i by wavefront blk_wave(i)) -----------
  // Loads are unconditional: a key index past the range is clamped to the last
  // key of the range (a valid, finite row), and its score is masked by `keep`
  // below, so its weight is exactly 0. No exec-masked branches means the
  // compiler can keep every load of a block in flight at once.
  // With four wavefronts the next block's K/V are loaded while this one is
  // computed (at D = 512 the second buffer lives in the accumulation
  // registers); with eight (two per SIMD) each wavefront has one block in
  // flight: two 32 KiB head-512 blocks per lane set do not fit the 256
  // registers a wavefront gets at two per SIMD, and the SIMD's two wavefronts
  // keep two blocks in flight between them.
  struct Blk {
    BiasT bias[E];
    int32_t kj;
    bf16x8 k[KSTEPS];
    bf16x8 v[NV];
  };
  // Issue order matters: loads retire in order, so the small bias / kind loads
  // go first (waiting for them does not wait for K and V), then K (needed by
  // the matrix cores first), then V.
  auto load_blk = [&](int j0, Blk& bl) {
    const int jk = min(j0 + qrow, my_hi - 1);
    bl.kj = 0;
    if constexpr (!kRules) {
#pragma unroll
      for (int e = 0; e < E; ++e) bl.bias[e] = biasb[(int64_t)row_s[e] * T + jk];
    } else {
      // branch-free: without kinds the load reads the first word of the K
      // row loaded below (no extra traffic) and its value is not used
      const int32_t kraw = *(kindb ? kindb + jk : (const int32_t*)(kbase + (int64_t)jk * D));
      bl.kj = kindb ? kraw : 0;
    }
    const __bf16* kp = kbase + (int64_t)jk * D + 8 * kgrp;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) bl.k[i] = ld_stream<bf16x8>(kp + 32 * i);
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int jv = min(j0 + it * KPI + vkey, my_hi - 1);
      bl.v[it] = ld_stream<bf16x8>(vbase + (int64_t)jv * DV + vd);
    }
  };
  const int stride = 16 * kDecWaves;
  // one 16-key block: S = Q K^T, online softmax, O += P V
  auto compute_blk = [&](const int j0, const Blk& cur) {
    const int jk = j0 + qrow;
    const bool kin = jk < my_hi;
    const bf16x8* kb = cur.k;
    const bf16x8* vv = cur.v;
    // bias / rules for the rows of this lane at key jk
    float badd[E];
    bool keep[E];
    const int32_t kj = cur.kj;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      badd[e] = 0.f;
      if constexpr (kRules) {
        keep[e] = row_ok[e] && kin && rules[e].allowed(jk, kj);
      } else {
        // branch-free, so the bias loads stay at the head of the block's loads
        const BiasT bv = cur.bias[e];
        keep[e] = row_ok[e] & kin & bias_live_bits<BiasT>(bv);
        badd[e] = bias_value<BiasT>(bv) * kLog2e;   // only read where keep[e]
      }
    }
    // S = Q K^T on the matrix cores
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      bf16x8 a;
      if constexpr (kQinLds)
        a = (qrow < R) ? *reinterpret_cast<const bf16x8*>(&s_q[qrow * D + 32 * i + 8 * kgrp]) : bf16x8{};
      else
        a = qa[i];
      acc = mfma16x16x32(a, kb[i], acc);
    }

    // softcap (0 = none) acts on scale * q.k before the bias is added: the raw
    // scores become the capped base-2 scores and the multiplier below 1
    float sl = scale_log2;
    if (cap_on) {
      asm volatile("" ::: "memory");   // a real branch, not selects on every block
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = softcap_base2(acc[e], cap2, scale_over_cap);
      sl = 1.f;
    }
    // online softmax on the S layout: lane = key (lane % 16), rows 4*kgrp + e
    float x[E];
    bool need_any = false;
    float alpha[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      x[e] = keep[e] ? fmaf(acc[e], sl, badd[e]) : -INFINITY;
      const float mt = row16_max(x[e]);
      const float mn = fmaxf(m_run[e], mt);
      const bool need = mn > m_run[e] + kRescaleThreshold;
      alpha[e] = need ? fast_exp2(m_run[e] - mn) : 1.f;
      if (need) m_run[e] = mn;
      need_any |= need;
    }
    if (__any(need_any)) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        l_run[e] *= alpha[e];
        const int r = 4 * kgrp + e;
        if (qrow == 0 && r < NR) s_alpha[w][r] = alpha[e];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float a = s_alpha[w][r];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[r][c] *= a;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float pe = (x[e] == -INFINITY) ? 0.f : fast_exp2(x[e] - m_run[e]);
      l_run[e] += pe;
      const int r = 4 * kgrp + e;
      if (r < NR) s_p[w][qrow][r] = pe;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // O += P V on the vector ALU (fp32)
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int jj = it * KPI + vkey;
      float pw[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) pw[r] = s_p[w][jj][r];
      const u32x4 raw = __builtin_bit_cast(u32x4, vv[it]);
      float vf[8];
      vf[0] = bf16lo(raw.x); vf[1] = bf16hi(raw.x);
      vf[2] = bf16lo(raw.y); vf[3] = bf16hi(raw.y);
      vf[4] = bf16lo(raw.z); vf[5] = bf16hi(raw.z);
      vf[6] = bf16lo(raw.w); vf[7] = bf16hi(raw.w);
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[r][c] = fmaf(pw[r], vf[c], o[r][c]);
    }
    __builtin_amdgcn_wave_barrier();  // s_p is rewritten by the next block
  };

  if constexpr (kPrefetch) {
    // two named buffers, alternating: the next block's loads are in flight
    // while this one is computed, with no register copies between them
    // The prefetch is unconditional: past the end of the range every key
    // clamps to the last row of the range (one cached row), and a
    // conditional load would make the wait counts at the join cover both
    // paths, i.e. wait for the prefetch too.
    Blk A, B;
    int j0 = my_lo + 16 * w;
    if (j0 < my_hi) load_blk(j0, A);
    if constexpr (kStep) {
      // after the first block's loads (the compiler would otherwise hoist the
      // stores above them): see side_stores
      asm volatile("" ::: "memory");
      reader_stores(1);
      side_stores();
    }
    while (j0 < my_hi) {
      const int j1 = j0 + stride;
      load_blk(j1, B);
      compute_blk(j0, A);
      if (j1 >= my_hi) break;
      const int j2 = j1 + stride;
      load_blk(j2, A);
      compute_blk(j1, B);
      j0 = j2;
    }
  } else {
    const int i_end = (!kTwoPerSimd || w >= 4) ? n_blk : n_old;
    const int i_step = kTwoPerSimd ? 4 : NW;
    for (int i = kTwoPerSimd && w >= 4 ? n_old + w - 4 : w; i < i_end; i += i_step) {
      const int j0 = my_lo + 16 * i;
      Blk A;
      load_blk(j0, A);
      compute_blk(j0, A);
    }
    side_stores();   // (a test in this loop costs more than the stores' wait)
  }

  // ---- 4. merge the wavefronts of this workgroup ----------------------------
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float lt = row16_sum(l_run[e]);
    const int r = 4 * kgrp + e;
    if (qrow == 0 && r < NR) { s_m[w][r] = m_run[e]; s_l[w][r] = lt; }
  }
  // lanes sharing a d-chunk hold different keys: sum them
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = o[r][c];
      if constexpr (KPI >= 2) v += lane_xor(v, 32);
      if constexpr (KPI >= 4) v += lane_xor(v, 16);
      if constexpr (KPI >= 8) v += lane_xor(v, 8);
      o[r][c] = v;
    }
  __syncthreads();
  float m_wg[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) mm = fmaxf(mm, s_m[ww][r]);
    m_wg[r] = mm;
  }
  // ---- 5. sum the waves in a fixed order (bit-reproducible), write the partial
  float* part = p.ws_part + ((int64_t)hk * S + rank) * PART;
  __shared__ float s_lrow[NR];
  if (tid < NR) {
    const int r = tid;
    float lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float f = (m_wg[r] == -INFINITY) ? 0.f : fast_exp2(s_m[ww][r] - m_wg[r]);
      lsum += s_l[ww][r] * f;
    }
    s_lrow[r] = lsum;
  }
  if constexpr (kParMerge) {
    if (lane < LPR) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float f = (m_wg[r] == -INFINITY) ? 0.f : fast_exp2(s_m[w][r] - m_wg[r]);
        float* dst = &s_o[(w * NR + r) * DV + vd];
#pragma unroll
        for (int c = 0; c < 8; ++c) dst[c] = o[r][c] * f;
      }
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      if (w == ww && lane < LPR) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float f = (m_wg[r] == -INFINITY) ? 0.f : fast_exp2(s_m[w][r] - m_wg[r]);
          float* dst = &s_o[r * DV + vd];
#pragma unroll
          for (int c = 0; c < 8; ++c) dst[c] = fmaf(o[r][c], f, dst[c]);
        }
      }
      __syncthreads();
    }
  }
  // this workgroup's O at item i (row 4i / DV, 4 values of d from 4i % DV)
  auto part_o = [&](int i) {
    f32x4 acc = reinterpret_cast<const f32x4*>(s_o)[i];
    if constexpr (kParMerge) {
#pragma unroll
      for (int ww = 1; ww < kDecWaves; ++ww) acc += reinterpret_cast<const f32x4*>(s_o + ww * NR * DV)[i];
    }
    return acc;
  };
  // a row with a single split: its partial is the result, written directly
  // with the arithmetic the merge below applies to one record (bit-identical)
  if (nsp == 1) {
    for (int i = tid; i < NR * DV / 4; i += kDecThreads) {
      const int r = (4 * i) / DV, d0 = (4 * i) % DV;
      if (r >= R) continue;
      const f32x4 a = part_o(i);
      const float mm = m_wg[r];
      const float fs = (mm == -INFINITY) ? 0.f : fast_exp2(mm - mm);
      const float den = 0.f * 0.f + s_lrow[r] * fs;
      float num[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) num[c] = 0.f * 0.f + a[c] * fs;
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const int s = r / G, g = r % G;
      uint16_t* op = (uint16_t*)p.out + (((b * p.Hq + hk * G + g) * p.S_q + s) * (int64_t)DV) + d0;
      u32x2 pk;
      pk.x = pack_bf16x2(num[0] * inv, num[1] * inv);
      pk.y = pack_bf16x2(num[2] * inv, num[3] * inv);
      *reinterpret_cast<u32x2*>(op) = pk;
    }
    return;
  }
  for (int i = tid; i < NR * DV / 4; i += kDecThreads) st_agent4(part + 4 * i, part_o(i));
  if (tid < NR) {
    st_agent(part + NR * DV + tid, m_wg[tid]);
    st_agent(part + NR * DV + NR + tid, s_lrow[tid]);
  }

  // ---- 6. the row's last split merges the row's records ---------------------
  // Each wavefront waits until its record stores are complete, then the
  // workgroup counts one arrival for its (kv head, b). The workgroup that finds
  // nsp - 1 arrivals before its own merges the nsp records in split order (the
  // same arithmetic, hence the same bits, whichever workgroup it is) and sets
  // the count back to zero for the next call:
  //   m = max m_i,  y = sum 2^(m_i - m) O_i / sum 2^(m_i - m) l_i
  // (a split that saw no live key has m_i = -inf and drops out; no live key at
  // all gives y = 0).
  __shared__ int s_arrived;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* const cnt = p.arrive + hk * p.B + b;
  if (tid == 0) s_arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_arrived != nsp - 1) return;
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float* parts = p.ws_part + ((int64_t)hk * S + first) * PART;
  constexpr int NQ = DV / 4;   // 4-float chunks of a row
  for (int it = tid; it < R * NQ; it += kDecThreads) {
    const int r = it / NQ, d0 = (it - r * NQ) * 4;
    // one pass, rescaled on the fly (running max); the records of 4 splits
    // are loaded together
    float mm = -INFINITY, den = 0.f;
    float num[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < nsp; sp0 += 4) {
      float pm[4], pl[4], pa[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* ps = parts + (int64_t)min(sp0 + u, nsp - 1) * PART;
        pm[u] = ld_agent(ps + NR * DV + r);
        pl[u] = ld_agent(ps + NR * DV + NR + r);
        ld_agent2(ps + r * DV + d0, pa[u][0], pa[u][1]);
        ld_agent2(ps + r * DV + d0 + 2, pa[u][2], pa[u][3]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (sp0 + u < nsp) {
          const float mn = fmaxf(mm, pm[u]);
          const float fo = (mm == -INFINITY) ? 0.f : fast_exp2(mm - mn);
          const float fs = (pm[u] == -INFINITY) ? 0.f : fast_exp2(pm[u] - mn);
          den = den * fo + pl[u] * fs;
#pragma unroll
          for (int c = 0; c < 4; ++c) num[c] = num[c] * fo + pa[u][c] * fs;
          mm = mn;
        }
      }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int s = r / G, g = r % G;
    uint16_t* op = (uint16_t*)p.out + (((b * p.Hq + hk * G + g) * p.S_q + s) * (int64_t)DV) + d0;
    u32x2 pk;
    pk.x = pack_bf16x2(num[0] * inv, num[1] * inv);
    pk.y = pack_bf16x2(num[2] * inv, num[3] * inv);
    *reinterpret_cast<u32x2*>(op) = pk;
  }
}

}  // namespace abgqa
