#pragma once
// bf16 prefill attention with a direct-to-LDS tile pipeline (gfx950).
//
// Same computation as attn_prefill.hip: onnxruntime skill
// "cuda-attention-kernel-patterns", section 4 (scale * QK^T, + bias, softmax,
// times V), section 6 (rows with no allowed key write zeros; masked keys are
// removed by selection), section 11 (external cache: keys are the slots below
// nonpad_kv_seqlen); mobius issue #366 (the float bias carries the causal,
// window, block-overlay and padding rules); query head h reads KV head h / G
// (onnxruntime PR #28242, CPU GQA excerpt).
//
// What differs is how tiles reach LDS. Here every byte a tile needs - K and V
// rows, and the tile's bias rows (or slot kinds) - is fetched with
// global_load_lds_dwordx4 (RW = 32: the workgroup's Q rows too): each lane names a 16-byte global chunk and the
// hardware writes the wavefront's 64 chunks to 1 KiB of consecutive LDS bytes
// (lane i at base + 16*i). No vector registers hold tile data, so nothing in
// the loop makes the compiler wait on a load, and NSTAGE tiles are in flight:
//
//   prologue   fetch tiles 0 .. NSTAGE-2
//   tile t     wait until this wavefront's fetches of tile t have landed
//              (s_waitcnt vmcnt: the fetches of the NSTAGE-2 younger tiles may
//              still be in flight), barrier (every wavefront's part of tile t
//              is in LDS, and every wavefront is done with tile t-1), fetch
//              tile t+NSTAGE-1 into the stage tile t-1 used, compute tile t.
//
// Every wavefront issues the same number of fetches per stage (surplus bias or
// kind fetches repeat one of identical bytes to the same place), so the wait
// count is a compile-time constant.
// Fetch indices past the end of the live list re-fetch the last live tile into
// a stage nobody reads. Keys at or beyond nonpad are fetched from row
// nonpad - 1 (a valid, finite row) and masked by selection, so the bits of
// the slots past nonpad are never read.
//
// The swizzle of the K/V tiles is the one attn_prefill.hip uses: LDS chunk
// position c of row r holds global chunk c ^ swz_bits<D>(r), so a wavefront
// fetching one row's chunks in order writes them permuted, for free.
//
// RW = 32: 32-row wavefronts on 32x32x16 MFMAs; RW = 16: 16-row wavefronts on
// 16x16x32 MFMAs. The B operand of S^T (the wavefront's Q^T fragments) sits in
// registers (kQReg) or, RW = 32 only, in an LDS Q tile, which leaves a lane's
// registers to the O^T accumulators when those must share the 256 ordinary
// vector registers. With 32-row wavefronts each K/V byte read from LDS serves
// twice the flops, and a 4-wavefront workgroup (128 rows) fetches each tile
// once for twice the rows; for D = 512 that needs Q^T in registers (128) and
// O^T in the accumulation registers (256). The compute per tile is that of
// attn_prefill.hip.
//
// V may have its own head size DV (the output rows are DV wide): a V tile
// holds DV-wide rows, swizzled by swz_bits<DV>, and O^T has DV / RW blocks.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "prefill_common.h"

namespace abgqa {

namespace {

// One wavefront-wide 16-byte-per-lane fetch into LDS at lds_wave_base (wave-
// uniform) + 16 * lane. Issued as inline asm on purpose: the compiler tracks
// its own direct-to-LDS loads and, unable to tell which LDS bytes they write,
// waits for all of them before any later LDS read - which would drain the
// whole pipeline every tile. Every wait for these fetches is the explicit
// s_waitcnt below. M0 carries the LDS address (one wait state after writing
// it) and is restored afterwards.
__device__ __forceinline__ void dma16(const void* gsrc, const unsigned char* lds_wave_base) {
  // wave-uniform by construction; readfirstlane makes that visible to the
  // compiler, which must place it in a scalar register
  const unsigned lds = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)((__attribute__((address_space(3))) const unsigned char*)lds_wave_base));
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(lds));
}

// The same fetch, non-temporal: for data read once (a workgroup's Q rows),
// which should not push the K/V tiles other workgroups still fetch out of the
// caches.
__device__ __forceinline__ void dma16_stream(const void* gsrc, const unsigned char* lds_wave_base) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)((__attribute__((address_space(3))) const unsigned char*)lds_wave_base));
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gsrc), "s"(lds));
}

// The same fetch from a wave-uniform base address plus a per-lane 32-bit byte
// offset (the scalar-base form: no per-lane address arithmetic).
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff,
                                        const unsigned char* lds_wave_base) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)((__attribute__((address_space(3))) const unsigned char*)lds_wave_base));
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds));
}

// The same with the LDS destination given as a 32-bit LDS address.
__device__ __forceinline__ void dma16_sl(const void* sbase, unsigned voff, unsigned lds_wave_base) {
  const unsigned lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds));
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier without the memory fences of __syncthreads (which would
// wait for every outstanding fetch); the asm statements keep the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 32-bit LDS address of a generic pointer into shared memory
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)((__attribute__((address_space(3))) const void*)p);
}

// LDS reads at base + cofs. Bases are masked to 20 bits where they are formed
// (LDS addresses are below 160 KiB), so the compiler knows base + cofs cannot
// wrap and puts a constant cofs into the instruction's offset field instead of
// adding it in a vector register for every read.
template <typename T>
__device__ __forceinline__ T lds_at(unsigned base, unsigned cofs) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>((size_t)(base + cofs));
}
__device__ __forceinline__ u32x2 lds_tr16_at(unsigned base, unsigned cofs) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>((size_t)(base + cofs)));
  return __builtin_bit_cast(u32x2, v);
}
constexpr unsigned kLdsMask = (1u << 20) - 1;

constexpr int kLdsBudget = 160 * 1024 - 6 * 1024;   // stages; the rest: live list

// O^T in the accumulation registers (32-row wavefronts at D = 512, where O^T
// takes all 256 of them and the S^T accumulator must stay in the ordinary
// registers, which no single choice of the compiler allows): the PV products
// are issued as inline asm on "a" operands, so each accumulator lives in the
// accumulation registers from its zeroing to its final read. The compiler sees
// no matrix-core op in that asm and so inserts no wait states for it; the
// ordering below provides them: two MFMAs into one accumulator are DV / 32
// MFMAs apart (16, or 8 at DV = 256, each of 8 passes), every VALU access
// to the accumulators (the rare rescale, the final read) first passes
// acc_settle, 32 wait states after the last MFMA, and the VALU-built P^T
// operands pass an s_nop that takes them as operands before the first PV MFMA.
__device__ __forceinline__ void mfma32x32x16_acc(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void acc_pin(f32x16& c) { asm volatile("" : "+a"(c)); }
__device__ __forceinline__ void acc_settle(f32x16 (&o)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
                 "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
}
__device__ __forceinline__ void acc_settle(f32x16 (&o)[8]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]));
}

// Chunk permutation of a bias row in the LDS bias stage: rows 256 bytes apart
// (4 bf16 rows or 2 fp32 rows of a 32-key tile) get different chunk orders.
template <typename BiasT>
__device__ __forceinline__ int bias_swz(int r) {
  constexpr int BROW = kTileKeys * (int)sizeof(BiasT);   // bytes per row
  return (r / (256 / BROW)) & (BROW / 16 - 1);
}
// element offset, within its row, of key k of the tile in that layout
template <typename BiasT>
__device__ __forceinline__ int bias_pos(int r, int k) {
  constexpr int EPV = 16 / (int)sizeof(BiasT);
  return ((k / EPV) ^ bias_swz<BiasT>(r)) * EPV + k % EPV;
}

template <int D, int RW, int NW, bool kRules, typename BiasT, bool kQReg, int KS, int DV = D>
struct DmaGeom {
  static_assert(kQReg || RW == 32, "an LDS Q tile needs 32-row wavefronts");
  static_assert(KS == 1 || (KS == 2 && kQReg && NW % 2 == 0), "key halves: Q^T in registers");
  static constexpr int TILE_K = kTileKeys * D * 2;             // one K tile
  static constexpr int TILE_V = kTileKeys * DV * 2;            // one V tile
  static constexpr int NKI = TILE_K / 1024;                    // fetches per K tile
  static constexpr int NVI = TILE_V / 1024;                    // fetches per V tile
  static constexpr int MQ_MAX = RW * NW / KS / 2;              // query tokens, G >= 2
  static constexpr int BROW = kTileKeys * (int)sizeof(BiasT);  // bias bytes per row per tile
  static constexpr int MASK_BYTES = kRules ? 1024 : ((MQ_MAX * BROW + 1023) / 1024) * 1024;
  static constexpr int NMI = MASK_BYTES / 1024;                // fetches for bias / kinds
  static constexpr int PW = (NKI + NVI) / NW + (NMI + NW - 1) / NW;  // fetches per wavefront per stage
  static constexpr int STAGE_BYTES = TILE_K + TILE_V + MASK_BYTES;
  // !kQReg: the workgroup's Q rows live in LDS (the B operand of S^T is read
  // from there)
  static constexpr bool kQLds = !kQReg;
  static constexpr int Q_BYTES = kQLds ? RW * NW * D * 2 : 0;
  static constexpr int NSTAGE0 = (kLdsBudget - Q_BYTES) / STAGE_BYTES;
  static constexpr int NSTAGE1 = NSTAGE0 > 4 ? 4 : NSTAGE0;
  static constexpr int NSTAGE = NSTAGE1 - NSTAGE1 % KS;   // whole super-stages of KS tiles
  static_assert(NSTAGE / KS >= 2, "two super-stages must fit");
  static_assert(KS * PW * (NSTAGE / KS - 2) <= 63, "wait count");
  // KS = 2: the key halves merge through the stage area
  static_assert(KS == 1 || (NW / KS) * (DV / RW * (RW == 32 ? 16 : 4) + 2) * 64 * 4 <= NSTAGE * STAGE_BYTES,
                "merge area");
};

}  // namespace

static_assert(kDmaMaxSeq / 1024 <= 128, "map words of the longest cache: one per thread");
template <int D, int RW, int NW, bool kRules, typename BiasT, bool kQReg, int KS, int DV = D>
__global__ __launch_bounds__(NW * 64) void attn_prefill_dma_kernel(AttnParams p, int n_qt) {
  using Geo = DmaGeom<D, RW, NW, kRules, BiasT, kQReg, KS, DV>;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;                 // 16-byte chunks per Q/K row
  constexpr int CPRV = DV / 8;               // 16-byte chunks per V row
  constexpr int NSTAGE = Geo::NSTAGE;
  constexpr int TILE_K = Geo::TILE_K;
  constexpr int TILE_V = Geo::TILE_V;
  constexpr int STAGE_BYTES = Geo::STAGE_BYTES;
  constexpr int MASK_BYTES = Geo::MASK_BYTES;
  constexpr int NKI = Geo::NKI;
  constexpr int NVI = Geo::NVI;
  constexpr int PW = Geo::PW;
  constexpr int KSTEPS = RW == 32 ? D / 16 : D / 32;   // k-steps of S^T over the head dim
  constexpr int DBLK = DV / RW;                        // d blocks of O^T
  constexpr bool kQLds = Geo::kQLds;
  constexpr int Q_BYTES = Geo::Q_BYTES;
  // O^T via mfma32x32x16_acc where O^T and Q^T of 32 rows do not fit the
  // ordinary registers together
  constexpr bool kAsmAcc = kQReg && RW == 32 && (D >= 512 || DV >= 512);
  static_assert(!(kAsmAcc && KS > 1), "key halves with accumulation-register O^T");
  constexpr int NSUP = NSTAGE / KS;   // super-stages: KS tiles each
  // The next stage's fetches go out in kFG groups spread over the S^T MFMAs of
  // the tile instead of all at its start: a wavefront that issues a whole
  // stage at once stalls until the memory pipeline has taken most of it, with
  // the matrix cores idle.
#ifndef ABGQA_FETCH_GROUPS
#define ABGQA_FETCH_GROUPS 4
#endif
  constexpr int kFG = ABGQA_FETCH_GROUPS < KSTEPS ? ABGQA_FETCH_GROUPS : KSTEPS;

  extern __shared__ __align__(16) unsigned char smem[];
  if constexpr (kQReg && RW == 32) {
    // An operand in an accumulation register: the compiler then keeps the
    // matrix-core accumulators in those registers (otherwise it assumes this
    // kernel uses none and forms the accumulators in the ordinary registers,
    // where O^T and Q^T of 32 rows do not fit together).
    asm volatile("" ::"a"(0));
  }
  const int T = p.T, G = p.G;
  const int n_kt_max = num_tiles(T);
  unsigned char* const stages = smem + Q_BYTES;   // [Q tile][stage 0][stage 1]...
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(stages + (size_t)NSTAGE * STAGE_BYTES);
  const int n_words = (n_kt_max + 31) / 32;
  uint16_t* s_list = reinterpret_cast<uint16_t*>(s_bits + n_words);
  __shared__ int s_nlive;
  __shared__ int s_nhalf[2];
  __shared__ int32_t s_ids[4];
  __shared__ int s_nids;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // KS = 2: wavefronts w and w + NW/2 hold the same rows (row group w % (NW/2))
  // and take alternate live tiles (key half kh), merged at the end
  constexpr int NWR = NW / KS;   // row groups
  const int rg = w % NWR, kh = w / NWR;

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = n_qt - 1 - (wg % n_qt);   // later (heavier) query tiles first
  const int bh = wg / n_qt;
  const int hk = bh % p.Hkv;
  const int64_t b = bh / p.Hkv;
  const int np = (int)clamp_nonpad(p.nonpad[b], T);
  const int MQ = (RW * NWR) / G;
  const int s0 = qt * MQ;
  const int s_end = min(s0 + MQ, p.S_q);
  const int n_kt = num_tiles(np);

  // ---- 1. this lane's query row (RW = 32: row 32*w + (l % 32); RW = 16: row
  // 16*w + (l % 16)). kQReg keeps its Q^T fragments (k-chunk 2*i + l/32, or
  // 4*i + l/16) in registers, loaded first so that the live-list scan's waits
  // cover them. ----
  const int col = lane & (RW - 1);
  const int grp = lane / RW;
  const int r = RW * rg + col;
  const int sl = r / G, g = r % G;
  const int s = s0 + sl;
  const bool row_ok = (r < MQ * G) && (s < p.S_q);
  const int h = hk * G + g;
  // this workgroup's words of the live-tile map (bias variant with a
  // workspace), loaded before anything waits so that they share the first
  // memory round trip with Q (n_words <= kDmaMaxSeq / 1024 = 64 <= NT)
  const uint32_t* map_row =
      (!kRules && p.tilemap) ? p.tilemap + ((size_t)(b * n_qt + qt)) * n_words : nullptr;
  const uint32_t map_pre = (map_row && tid < n_words) ? map_row[tid] : 0u;
  bf16x8 qf[kQLds ? 1 : KSTEPS];
#ifndef ABGQA_QSTAGE
#define ABGQA_QSTAGE 1
#endif
  constexpr bool kQStage = !kQLds && RW == 32 && ABGQA_QSTAGE && NW * RW * D * 2 <= NSTAGE * STAGE_BYTES;
  if constexpr (kQStage) {
    // 32-row wavefronts: each wavefront copies its 32 Q rows whole into its
    // own part of the (still unused) stage area with direct-to-LDS fetches (a
    // row's chunks contiguous, swizzled like the K tiles) and reads its Q^T
    // fragments from there: the global reads are whole rows instead of 32-byte
    // pieces of 32 rows per instruction. Rows past the chunk copy a valid row
    // (finite; their outputs are never stored). Only where the workgroup's Q
    // rows fit in the stage area (not with D = 512 beside DV = 256).
    constexpr int RPF = 64 / CPR;   // Q rows per fetch
    unsigned char* const qw = stages + (size_t)w * RW * D * 2;
#pragma unroll
    for (int k = 0; k < RW / RPF; ++k) {
      const int rl = k * RPF + lane / CPR, cc = lane % CPR;
      const int rq = RW * rg + rl;
      const int sq = min(s0 + rq / G, p.S_q - 1);
      const __bf16* src = (const __bf16*)p.q + ((b * p.Hq + hk * G + rq % G) * p.S_q + sq) * (int64_t)D;
      dma16_stream(src + 8 * (cc ^ swz_bits<D>(rl)), qw + k * 1024);   // long prefill 337.6 -> 332.0 us
    }
    wait_vmcnt<0>();
    const unsigned qb = lds_addr(qw) & kLdsMask;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      const int c = 2 * i + grp;
      qf[i] = lds_at<bf16x8>(qb, (unsigned)(col * D * 2 + 16 * ((c & ~15) | ((c & 15) ^ swz_bits<D>(col)))));
    }
  } else if constexpr (!kQLds) {
    const __bf16* qp = (const __bf16*)p.q + ((b * p.Hq + h) * p.S_q + (row_ok ? s : 0)) * (int64_t)D;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i)
      qf[i] = row_ok ? ld_global<bf16x8>(qp + 8 * ((RW == 32 ? 2 : 4) * i + grp)) : bf16x8{};
  }
  RowRule rule{};
  if constexpr (kRules) {
    if (row_ok) rule = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window, p.circular);
  }
  // the row's causal/window key interval for the whole-tile test of the rules
  // variant; a row past the chunk passes it (its output is never stored)
  const int rule_lo = row_ok ? rule.lo : INT_MIN, rule_hi = row_ok ? rule.hi : INT_MAX;
  // a circular cache's interval may wrap round into a second one
  const int rule_lo2 = row_ok ? rule.lo2 : INT_MIN, rule_hi2 = row_ok ? rule.hi2 : INT_MAX;

  // ---- 2. live tiles ---------------------------------------------------------
  // read from LDS, the count is the same in every lane: say so, so that the
  // loop below (and every LDS address derived from its counter) is scalar
  const int n_live = __builtin_amdgcn_readfirstlane(
      build_live_list<NT, kRules, BiasT>(p, b, np, s0, s_end, n_kt, s_bits, s_list, n_words, s_ids,
                                         &s_nids, &s_nlive, map_row, map_pre));
  // KS = 2: the live tiles split by parity of their key tile, even tiles for
  // key half 0 (s_list[0, ...)), odd ones for half 1 (s_list[khalf, ...)), so
  // a fully masked tile that one variant lists and another skips changes no
  // other tile's half (it only adds exact zeros to its own)
  const int khalf = (n_kt_max + 1) / 2;
  int n_h0 = n_live, n_h1 = 0;
  if constexpr (KS == 2) {
    if (w == 0) {
      int be = 0, bo = 0;
      for (int t0 = 0; t0 < n_kt; t0 += 64) {
        const int t = t0 + lane;
        const bool live = (t < n_kt) && ((s_bits[t >> 5] >> (t & 31)) & 1u);
        const uint64_t me = __ballot(live && !(t & 1)), mo = __ballot(live && (t & 1));
        const uint64_t below = (1ull << lane) - 1ull;
        if (live) {
          if (t & 1) s_list[khalf + bo + __popcll(mo & below)] = (uint16_t)t;
          else s_list[be + __popcll(me & below)] = (uint16_t)t;
        }
        be += __popcll(me);
        bo += __popcll(mo);
      }
      if (lane == 0) { s_nhalf[0] = be; s_nhalf[1] = bo; }
    }
    __syncthreads();
    n_h0 = __builtin_amdgcn_readfirstlane(s_nhalf[0]);
    n_h1 = __builtin_amdgcn_readfirstlane(s_nhalf[1]);
  }
  // nothing may be pending in registers once the pipeline starts: every wait
  // in the loop below is the explicit one
  wait_vmcnt<0>();

  const float scale_log2 = p.scale * kLog2e;
  const bool cap_on = p.softcap > 0.f;
  const float cap2 = p.softcap * kLog2e, scale_over_cap = cap_on ? p.scale / p.softcap : 0.f;
  const __bf16* kg = (const __bf16*)p.k + (b * p.Hkv + hk) * (int64_t)T * D;
  const __bf16* vg = (const __bf16*)p.v + (b * p.Hkv + hk) * (int64_t)T * DV;
  const int32_t* kindb = p.slot_kind ? p.slot_kind + b * T : nullptr;
  // rules variant: the kind stage is read unconditionally (it holds K bytes
  // when there are no slot kinds) and masked to kind 0 then, so no branch
  // separates these reads from the K reads they are scheduled with
  const int32_t kind_mask = kindb ? -1 : 0;
  const BiasT* biasb = kRules ? nullptr : (const BiasT*)p.bias + b * p.S_q * (int64_t)T;

  // ---- 3. one stage's fetches ----------------------------------------------
  // Wavefront w fetches K rows [w*KPW*RPI, (w+1)*KPW*RPI) of the tile, V rows
  // [w*VPW*RPIV, (w+1)*VPW*RPIV), and its share of the bias rows (or the slot
  // kinds), so the kind of every fetch is known at compile time and the issue
  // is branch-free.
  constexpr int KPW = NKI / NW;            // K fetches per wavefront
  constexpr int VPW = NVI / NW;            // V fetches per wavefront
  constexpr int NMI = Geo::NMI;
  constexpr int MPW = (NMI + NW - 1) / NW;  // bias / kind fetches per wavefront
  constexpr int RPI = 64 / CPR;             // K rows per fetch
  constexpr int RPIV = 64 / CPRV;           // V rows per fetch
  static_assert(NKI % NW == 0 && NVI % NW == 0 && 64 % CPR == 0 && 64 % CPRV == 0 &&
                    PW == KPW + VPW + MPW,
                "fetch layout");
  // fetch order: K and V alternate while both have fetches left, then the
  // rest of the larger, then bias / kinds
  constexpr int NIL = KPW < VPW ? KPW : VPW;
  const int lrow = lane / CPR, lcc = lane % CPR;
  const int lrowv = lane / CPRV, lccv = lane % CPRV;
  // byte offsets of this lane's chunks from the tile's first K row / first V
  // row / first bias row / first slot kind
  unsigned kv_off[KPW], v_off[VPW];
#pragma unroll
  for (int k = 0; k < KPW; ++k) {
    const int kr = (w * KPW + k) * RPI + lrow;
    kv_off[k] = (unsigned)(kr * D + 8 * (lcc ^ swz_bits<D>(kr))) * 2u;
  }
#pragma unroll
  for (int k = 0; k < VPW; ++k) {
    const int vr = (w * VPW + k) * RPIV + lrowv;
    v_off[k] = (unsigned)(vr * DV + 8 * (lccv ^ swz_bits<DV>(vr))) * 2u;
  }
  // Bias rows sit in LDS with their 16-byte chunks permuted by bias_swz (row
  // r's chunk c at position c ^ bias_swz(r)): rows 256 bytes apart would
  // otherwise hit the same banks when the lanes of a wavefront read the rows
  // of their query tokens.
  unsigned m_off[MPW];
  int m_col[MPW];   // first key of the lane's chunk in its row
#pragma unroll
  for (int m = 0; m < MPW; ++m) {
    if constexpr (kRules) {
      m_off[m] = 16u * (unsigned)(lane & 7);    // lanes 8.. repeat lanes 0..7
      m_col[m] = 0;
    } else {
      constexpr int EPV = 16 / (int)sizeof(BiasT);
      constexpr int CB = Geo::BROW / 16;       // 16-byte chunks per bias row
      const int c = min(w * MPW + m, NMI - 1) * 64 + lane;
      const int lrow = c / CB;                 // the row in LDS
      const int row = min(s0 + lrow, p.S_q - 1) - s0;
      m_col[m] = ((c % CB) ^ bias_swz<BiasT>(lrow)) * EPV;
      m_off[m] = (unsigned)(row * T + m_col[m]) * (unsigned)sizeof(BiasT);
    }
  }
  // LDS layout of the stages: the K tiles of every stage, then the V tiles,
  // then the bias / kind blocks. A stage's tile lies a multiple of TILE_K (or
  // TILE_V) from stage 0's, so with the stage known at compile time (the loop below
  // runs NSTAGE tiles per iteration when NSTAGE == 2) a read of stage st
  // differs from one of stage 0 only in the instruction's offset field.
  const unsigned lds0 = lds_addr(stages);
  // fetch f of this wavefront's PW for the tile starting at key j0 into stage
  // st: f < KPW + VPW are K and V rows (f < 2*NIL: K for even f), the rest
  // bias rows or slot kinds. Rows at or past nonpad are fetched from row nonpad - 1, and bias /
  // kind chunks past the end of the cache from its last chunk; both clamps are
  // folded into the lane's offset, so the issue has no branch. f is a
  // compile-time constant at every call.
  auto fetch_one = [&](const int f, const int j0, const int st) {
    const int lim = np - 1 - j0;   // the tile's last valid row (j0 < nonpad)
    if (f < KPW + VPW) {
      const bool is_k = f < 2 * NIL ? (f & 1) == 0 : KPW > VPW;
      const int k = f < 2 * NIL ? f >> 1 : f - NIL;
      if (is_k) {
        const int ii = w * KPW + k;
        const int kr = ii * RPI + lrow;
        const unsigned off = kv_off[k] + (unsigned)(min(lim - kr, 0) * (2 * D));
        dma16_sl(kg + (int64_t)j0 * D, off, lds0 + st * TILE_K + ii * 1024);
      } else {
        const int ii = w * VPW + k;
        const int vr = ii * RPIV + lrowv;
        const unsigned off = v_off[k] + (unsigned)(min(lim - vr, 0) * (2 * DV));
        dma16_sl(vg + (int64_t)j0 * DV, off, lds0 + NSTAGE * TILE_K + st * TILE_V + ii * 1024);
      }
    } else {
      const int m = f - KPW - VPW;
      const int ii = min(w * MPW + m, NMI - 1);   // surplus fetches repeat the last one
      const unsigned dst = lds0 + NSTAGE * (TILE_K + TILE_V) + st * MASK_BYTES + ii * 1024;
      if constexpr (kRules) {
        const int c = 4 * (lane & 7);   // this lane's first slot kind
        const unsigned off = m_off[m] + (unsigned)(min(T - 4 - j0 - c, 0) * 4);
        dma16_sl(kindb ? (const void*)(kindb + j0) : (const void*)kg, off, dst);
      } else {
        constexpr int EPV = 16 / (int)sizeof(BiasT);
        const int col = m_col[m];   // this lane's first key in the row
        const unsigned off = m_off[m] + (unsigned)(min(T - EPV - j0 - col, 0) * (int)sizeof(BiasT));
        dma16_sl(biasb + (int64_t)s0 * T + j0, off, dst);
      }
    }
  };
  // first key of tile u of key half k (KS = 1: of the live list). Past the end
  // of a list: its last tile again; an empty half takes the other half's
  // tiles (fetched, never computed).
  auto key_of = [&](int k, int u) {
    int idx;
    if constexpr (KS == 1) {
      idx = min(u, n_live - 1);
    } else {
      const int kk = (k == 0 ? n_h0 : n_h1) > 0 ? k : 1 - k;
      idx = kk * khalf + min(u, (kk == 0 ? n_h0 : n_h1) - 1);
    }
    return __builtin_amdgcn_readfirstlane((int)s_list[idx] * kTileKeys);
  };
  auto fetch_stage = [&](int j0, int st) {
#pragma unroll
    for (int f = 0; f < PW; ++f) fetch_one(f, j0, st);
  };
  // the fetches of one super-stage (KS tiles: tile k from key jn[k] into stage
  // KS*ssn + k) in kFG groups: group g is [KS*PW*g/kFG, KS*PW*(g+1)/kFG)
  auto fetch_group = [&](const int g, const int* jn, const int ssn) {
#pragma unroll
    for (int f = KS * PW * g / kFG; f < KS * PW * (g + 1) / kFG; ++f)
      fetch_one(f % PW, jn[f / PW], KS * ssn + f / PW);
  };

  // ---- 4. main loop ---------------------------------------------------------
  using Acc = typename std::conditional<RW == 32, f32x16, f32x4>::type;
  Acc oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) {
    oacc[i] = Acc{};
    if constexpr (kAsmAcc) acc_pin(oacc[i]);
  }
  float m_run = -INFINITY, l_run = 0.f;

  if (n_live > 0) {
    if constexpr (kQLds) {
      // the workgroup's Q rows into the swizzled Q tile (row r = s_local*G + g,
      // clamped to a valid row past the chunk); older than every stage fetch,
      // so the first tile's wait covers them too
      constexpr int QPW = Q_BYTES / 1024 / NW;
#pragma unroll
      for (int k = 0; k < QPW; ++k) {
        const int ii = w * QPW + k;
        const int c = ii * 64 + lane;
        const int qr = c / CPR, cc = c % CPR;
        const int qs = min(s0 + qr / G, p.S_q - 1);
        const int qh = hk * G + qr % G;
        dma16((const __bf16*)p.q + ((b * p.Hq + qh) * p.S_q + qs) * (int64_t)D + 8 * (cc ^ swz_bits<D>(qr)),
              smem + ii * 1024);
      }
    }
#pragma unroll
    for (int u = 0; u < NSUP - 1; ++u)
#pragma unroll
      for (int k = 0; k < KS; ++k) fetch_stage(key_of(k, u), KS * u + k);
  }
  // Per-lane byte offsets into the swizzled tiles. Chunk c of row r sits at
  // 16 * (c ^ swz_bits<D>(r)) (V: swz_bits<DV>); the XOR touches only the low
  // SWB bits of c, so the reads of one lane need a few base offsets (by those
  // low bits of c) plus compile-time multiples of SPAN = 16 << SWB bytes.
  constexpr int SWB = swz_width<D>();
  constexpr int SPAN = 16 << SWB;
  constexpr int SWBV = swz_width<DV>();
  constexpr int SPANV = 16 << SWBV;
  // RW = 32: K/Q chunk 2*i + grp -> groups i % NKG; V chunk 4*blk + vdofs/8 ->
  // groups blk % NVG, times the two 8-row halves (the swizzle sees row bit 3).
  // RW = 16: K chunk 4*i + grp -> groups i % NKG; V chunk 2*blk + vdofs/8 ->
  // groups blk % NVG.
  constexpr int NKG = RW == 32 ? (1 << SWB) / 2 : (1 << SWB) / 4;
  constexpr int NVG = RW == 32 ? (1 << SWBV) / 4 : (1 << SWBV) / 2;
  unsigned k_lane[NKG];                  // K (and, RW = 32, Q) rows
  unsigned v_lane[RW == 32 ? 2 : 1][NVG];  // V^T transposing reads
  if constexpr (RW == 32) {
    // S^T: lane reads row col, chunk 2*i + grp
#pragma unroll
    for (int m = 0; m < NKG; ++m)
      k_lane[m] = (unsigned)(col * D * 2 + 16 * ((2 * m + grp) ^ swz_bits<D>(col)));
    // PV: lane 16*gq + 4*kq + jq reads row 16*step + 8*half + vkey0, d = 32*blk +
    // vdofs: chunk 4*blk + vdofs/8
    const int gq = lane >> 4, kq = (lane >> 2) & 3, jq = lane & 3;
    const int vkey0 = 4 * (gq >> 1) + kq;
    const int vdofs = 16 * (gq & 1) + 4 * jq;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int m = 0; m < NVG; ++m) {
        const int row = 8 * hf + vkey0;
        v_lane[hf][m] = (unsigned)(row * DV * 2 + 16 * ((4 * m + (vdofs >> 3)) ^ swz_bits<DV>(row)) +
                                   2 * (vdofs & 7));
      }
  } else {
    // S^T: row 16*kb + col, chunk 4*i + grp
#pragma unroll
    for (int m = 0; m < NKG; ++m)
      k_lane[m] = (unsigned)(col * D * 2 + 16 * ((4 * m + grp) ^ swz_bits<D>(col)));
    // PV: lane 16*g + 4*k + j reads row vkey0 (+16), d = 16*blk + vdofs:
    // chunk 2*blk + vdofs/8
    const int vkey0 = lane >> 2;
    const int vdofs = 4 * (lane & 3);
#pragma unroll
    for (int m = 0; m < NVG; ++m)
      v_lane[0][m] = (unsigned)(vkey0 * DV * 2 + 16 * ((2 * m + (vdofs >> 3)) ^ swz_bits<DV>(vkey0)) +
                                2 * (vdofs & 7));
  }
  // this wavefront's Q rows in the LDS Q tile, one base per k-chunk group
  unsigned q_base[kQLds ? NKG : 1];
  if constexpr (kQLds) {
    const unsigned qa0 = lds_addr(smem) + (unsigned)(RW * rg * D * 2);
#pragma unroll
    for (int m = 0; m < NKG; ++m) q_base[m] = (qa0 + k_lane[m]) & kLdsMask;
  }
  // loop-invariant read bases of stage 0 (stage st adds st * TILE_K, or
  // st * TILE_V)
  unsigned k_base[NKG], v_base[RW == 32 ? 2 : 1][NVG];
#pragma unroll
  for (int m = 0; m < NKG; ++m) k_base[m] = (lds0 + kh * TILE_K + k_lane[m]) & kLdsMask;
#pragma unroll
  for (int hf = 0; hf < (RW == 32 ? 2 : 1); ++hf)
#pragma unroll
    for (int m = 0; m < NVG; ++m)
      v_base[hf][m] = (lds0 + NSTAGE * TILE_K + kh * TILE_V + v_lane[hf][m]) & kLdsMask;

  // one tile from key j0, held by stage KS*ss + kh (super-stage ss); jn / ssn
  // name the super-stage whose fetches go out during its S^T MFMAs
  auto tile_step = [&](const int j0, const int ss, const int* jn, const int ssn)
                       __attribute__((always_inline)) {
    const bool full = j0 + kTileKeys <= np;   // no key of the tile at or past nonpad
    const unsigned char* ms = stages + NSTAGE * (TILE_K + TILE_V) + (KS * ss + kh) * MASK_BYTES;
    // stage offsets of K and V reads (the key half's kh * TILE_K or kh * TILE_V
    // is in the bases)
    const unsigned KO = (unsigned)(KS * ss * TILE_K);
    const unsigned VO = (unsigned)(KS * ss * TILE_V);

    if constexpr (RW == 32) {
      BiasT bvs[4][4];
      int32_t kvs[4][4];
      // S^T = K Q^T; lane l: query row l % 32, keys 8*i + 4*(l/32) + jj
      // fragments of k-step i + PD are read while the MFMA of step i runs. With
      // one wavefront per SIMD the LDS round trip, not the matrix core, sets the
      // pace of this phase, so the reads in flight decide it: 8 ahead is ~10%
      // faster over a whole D = 512 prefill than 4 (12 ahead is no better).
#ifndef ABGQA_PD32
#define ABGQA_PD32 8
#endif
      constexpr int PD = KSTEPS < ABGQA_PD32 ? KSTEPS : ABGQA_PD32;
      // NCH accumulation chains (k-step i into chain i % NCH), summed at the
      // end. Back-to-back dependent 32x32x16 MFMAs issue at the full rate on
      // this part, so one chain: its registers go to the deeper read-ahead.
#ifndef ABGQA_SCH32
#define ABGQA_SCH32 1
#endif
      constexpr int NCH = KSTEPS < ABGQA_SCH32 ? KSTEPS : ABGQA_SCH32;
      f32x16 schain[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) schain[c] = f32x16{};
      constexpr int NQR = kQLds ? 2 : 1;   // LDS reads per k-step
      bf16x8 ka[PD], qa[kQLds ? PD : 1];
#pragma unroll
      for (int i = 0; i < PD; ++i) {
        ka[i] = lds_at<bf16x8>(k_base[i % NKG], KO + SPAN * (i / NKG));
        if constexpr (kQLds) qa[i] = lds_at<bf16x8>(q_base[i % NKG], SPAN * (i / NKG));
      }
      __builtin_amdgcn_sched_group_barrier(0x100, NQR * PD, 0);
      // this lane's bias values (or slot kinds) for keys 8*i + 4*(l/32) + jj,
      // read behind the first K fragments (ahead of them they would take
      // places of the read-ahead) so their latency hides under the MFMAs
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kb = 8 * i + 4 * grp;
        if constexpr (kRules) {
          const int4 kk = *reinterpret_cast<const int4*>(ms + 4 * kb);
          *reinterpret_cast<int4*>(kvs[i]) = int4{kk.x & kind_mask, kk.y & kind_mask, kk.z & kind_mask, kk.w & kind_mask};
        } else {
          const BiasT* br = reinterpret_cast<const BiasT*>(ms) + sl * kTileKeys + bias_pos<BiasT>(sl, kb);
          if constexpr (sizeof(BiasT) == 2) *reinterpret_cast<u32x2*>(bvs[i]) = *reinterpret_cast<const u32x2*>(br);
          else *reinterpret_cast<u32x4*>(bvs[i]) = *reinterpret_cast<const u32x4*>(br);
        }
      }
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i) {
        const bf16x8 a = ka[i % PD];
        bf16x8 qb;
        if constexpr (kQLds) qb = qa[i % PD];
        else qb = qf[i];
        if (i + PD < KSTEPS) {
          ka[i % PD] = lds_at<bf16x8>(k_base[(i + PD) % NKG], KO + SPAN * ((i + PD) / NKG));
          if constexpr (kQLds) qa[i % PD] = lds_at<bf16x8>(q_base[(i + PD) % NKG], SPAN * ((i + PD) / NKG));
        }
        schain[i % NCH] = mfma32x32x16(a, qb, schain[i % NCH]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + PD < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, NQR, 0);
        constexpr int GS = KSTEPS / kFG;   // k-steps per fetch group
        if (kFG > 1 && i % GS == GS - 1 && i / GS + 1 < kFG) fetch_group(i / GS + 1, jn, ssn);
      }
      f32x16 sacc = schain[0];
#pragma unroll
      for (int c = 1; c < NCH; ++c) sacc += schain[c];
      // V^T fragments of the first PV MFMAs, read while the softmax runs.
      // MFMA u = 2*blk + step; lane 16*gq + 4*kq + jq reads
      // V[16*step + 8*half + 4*(gq/2) + kq][32*blk + 16*(gq%2) + 4*jq]
      constexpr int NU = 2 * DBLK;
#ifndef ABGQA_PVD32
#define ABGQA_PVD32 4
#endif
      constexpr int PVD = NU < ABGQA_PVD32 ? NU : ABGQA_PVD32;
      auto vread = [&](int u) {
        const int blk = u >> 1;
        const unsigned so = SPANV * (blk / NVG) + 16 * (u & 1) * DV * 2;
        const u32x2 lo = lds_tr16_at(v_base[0][blk % NVG], VO + so);
        const u32x2 hi = lds_tr16_at(v_base[1][blk % NVG], VO + so);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      };
      bf16x8 vf[PVD];
      if constexpr (!kAsmAcc) {
#pragma unroll
        for (int u = 0; u < PVD; ++u) vf[u] = vread(u);
      }
      // softcap (0 = none) on scale * q.k, before the bias: capped base-2 scores,
      // multiplier 1 (a real branch, not selects on every tile)
      float sl = scale_log2;
      if (cap_on) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = softcap_base2(sacc[e], cap2, scale_over_cap);
        sl = 1.f;
      }
      float x[16];
      float mt = -INFINITY;
      if constexpr (kRules) {
        // the common case: the tile lies inside every row's causal/window
        // interval (so below nonpad) and holds no pad slot (the OR of the kinds
        // is not negative), so every key is allowed, block or not, and no score
        // needs the per-element rule (a real branch; both sides give an
        // allowed score the same bits)
        int kor = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) kor |= kvs[i][jj];
        const bool inside = (j0 >= rule_lo && j0 + kTileKeys - 1 <= rule_hi) ||
                            (j0 >= rule_lo2 && j0 + kTileKeys - 1 <= rule_hi2);
        if (!__any(kor < 0 || !inside)) {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int e = 0; e < 16; ++e) x[e] = sacc[e] * sl;
        } else {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              // allowed() includes j < nonpad; a row past the chunk has no rule
              const int j = j0 + 8 * i + 4 * grp + jj;
              x[4 * i + jj] = rule.allowed(j, kvs[i][jj]) ? sacc[4 * i + jj] * sl : -INFINITY;
            }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            // a -inf bias gives -inf (the score is finite: every fetched key row
            // is a valid row); keys at or past nonpad only in a partial tile
            x[4 * i + jj] = fmaf(sacc[4 * i + jj], sl, bias_f32<BiasT>(bvs[i][jj]) * kLog2e);
          }
      }
      if constexpr (!kRules) {
        if (!full) {
          // the tile crossing nonpad: keys at or past it are not keys (a real
          // branch, taken at most once per workgroup)
          asm volatile("" ::: "memory");
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (j0 + 8 * (e >> 2) + 4 * grp + (e & 3) >= np) x[e] = -INFINITY;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) mt = fmaxf(mt, x[e]);
      mt = fmaxf(mt, lane_xor(mt, 32));
      const float mn = fmaxf(m_run, mt);
      const bool need = mn > m_run + kRescaleThreshold;
      const bool rescale = __any(need);
      float alpha = 1.f;
      if (rescale) {
        alpha = need ? fast_exp2(m_run - mn) : 1.f;
        if (need) m_run = mn;
        l_run *= alpha;
      }
      // 2^(-inf) = 0 for masked keys; a row with no live key yet subtracts 0
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      uint32_t pw[8];
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(x[e] - m_use);
        const float p1 = fast_exp2(x[e + 1] - m_use);
        const uint32_t pk = pack_bf16x2(p0, p1);
        lsum += bf16lo(pk) + bf16hi(pk);
        pw[e >> 1] = pk;
      }
      l_run += lsum;
      bf16x8 pb0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      bf16x8 pb1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
      if (rescale) {
        // rare (the running maximum rose by more than 8): a real branch - the
        // asm keeps the compiler from turning it into selects executed on every
        // tile, which would also pull the accumulators out of their registers
        asm volatile("" ::: "memory");
        if constexpr (kAsmAcc) {
          acc_settle(oacc);
#pragma unroll
          for (int blk = 0; blk < DBLK; ++blk) {
            oacc[blk] *= alpha;
            acc_pin(oacc[blk]);
          }
          asm volatile("s_nop 4");   // VALU writes before the next MFMA reads them
        } else {
#pragma unroll
          for (int blk = 0; blk < DBLK; ++blk) oacc[blk] *= alpha;
        }
      }
      // O^T += V^T P^T, fragments read PVD MFMAs ahead
      if constexpr (kAsmAcc) {
        // P^T comes from VALU instructions, and an MFMA reading a register that
        // a VALU instruction wrote needs two wait states in between, which the
        // compiler does not insert before an asm MFMA: this asm sits after the
        // last write of pb0 / pb1 (it takes them as operands) and provides them
        asm volatile("s_nop 1" : "+v"(pb0), "+v"(pb1));
        // the first key half of every d block, then the second half
        auto useq = [](int q) { return q < DBLK ? 2 * q : 2 * (q - DBLK) + 1; };
#pragma unroll
        for (int q = 0; q < PVD; ++q) vf[q] = vread(useq(q));
#pragma unroll
        for (int q = 0; q < NU; ++q) {
          const int u = useq(q);
          const bf16x8 va = vf[q % PVD];
          if (q + PVD < NU) vf[q % PVD] = vread(useq(q + PVD));
          mfma32x32x16_acc(oacc[u >> 1], va, (u & 1) ? pb1 : pb0);
        }
      } else {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const bf16x8 va = vf[u % PVD];
          if (u + PVD < NU) vf[u % PVD] = vread(u + PVD);
          oacc[u >> 1] = mfma32x32x16(va, (u & 1) ? pb1 : pb0, oacc[u >> 1]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (u + PVD < NU) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    } else {
      // this lane's bias values (or slot kinds) for keys 16*kb + 4*(l/16) + e,
      // read first so their latency hides under the S^T MFMAs
      BiasT bvs[2][4];
      int32_t kvs[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kf = 16 * kb + 4 * grp;
        if constexpr (kRules) {
          const int4 kk = *reinterpret_cast<const int4*>(ms + 4 * kf);
          *reinterpret_cast<int4*>(kvs[kb]) = int4{kk.x & kind_mask, kk.y & kind_mask, kk.z & kind_mask, kk.w & kind_mask};
        } else {
          const BiasT* br = reinterpret_cast<const BiasT*>(ms) + sl * kTileKeys + bias_pos<BiasT>(sl, kf);
          if constexpr (sizeof(BiasT) == 2) *reinterpret_cast<u32x2*>(bvs[kb]) = *reinterpret_cast<const u32x2*>(br);
          else *reinterpret_cast<u32x4*>(bvs[kb]) = *reinterpret_cast<const u32x4*>(br);
        }
      }
      // S^T = K Q^T in two 16-key halves; lane l: query row l % 16, keys
      // 16*kb + 4*(l/16) + e. The halves' MFMAs alternate: an MFMA that
      // accumulates onto the result of the one just issued waits for it to
      // finish, which halves the matrix-core rate of a single chain.
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      {
        constexpr int NS = 2 * KSTEPS;   // step n: k-step n / 2 of key half n % 2
        constexpr int PD = 8;            // K fragments read PD steps ahead of their MFMA
        auto kread = [&](int n) {
          const int i = n >> 1;
          return lds_at<bf16x8>(k_base[i % NKG], KO + SPAN * (i / NKG) + (n & 1) * 16 * D * 2);
        };
        bf16x8 ka[PD];
#pragma unroll
        for (int n = 0; n < PD; ++n) ka[n] = kread(n);
        __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          const bf16x8 a = ka[n % PD];
          if (n + PD < NS) ka[n % PD] = kread(n + PD);
          sacc[n & 1] = mfma16x16x32(a, qf[n >> 1], sacc[n & 1]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (n + PD < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          constexpr int GS = NS / kFG;   // steps per fetch group
          if (kFG > 1 && n % GS == GS - 1 && n / GS + 1 < kFG) fetch_group(n / GS + 1, jn, ssn);
        }
      }
      // V^T fragments of the first PV MFMAs, read while the softmax runs;
      // lane 16*gq + 4*kq + jq reads V[4*gq + kq (+16)][16*blk + 4*jq]
      constexpr int PVD = 4;
      auto vread = [&](int blk) {
        const unsigned so = SPANV * (blk / NVG);
        const u32x2 lo = lds_tr16_at(v_base[0][blk % NVG], VO + so);
        const u32x2 hi = lds_tr16_at(v_base[0][blk % NVG], VO + so + 16 * DV * 2);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      };
      bf16x8 vf[PVD];
#pragma unroll
      for (int u = 0; u < PVD; ++u) vf[u] = vread(u);
      float sl = scale_log2;
      if (cap_on) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[kb][e] = softcap_base2(sacc[kb][e], cap2, scale_over_cap);
        sl = 1.f;
      }
      float x[8];
      float mt = -INFINITY;
      if constexpr (kRules) {
        // the whole-tile test of the 32-row branch
        int kor = 0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) kor |= kvs[kb][e];
        const bool inside = (j0 >= rule_lo && j0 + kTileKeys - 1 <= rule_hi) ||
                            (j0 >= rule_lo2 && j0 + kTileKeys - 1 <= rule_hi2);
        if (!__any(kor < 0 || !inside)) {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * kb + e] = sacc[kb][e] * sl;
        } else {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[4 * kb + e] = rule.allowed(j0 + 16 * kb + 4 * grp + e, kvs[kb][e]) ? sacc[kb][e] * sl : -INFINITY;
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * kb + e] = fmaf(sacc[kb][e], sl, bias_f32<BiasT>(bvs[kb][e]) * kLog2e);
      }
      if constexpr (!kRules) {
        if (!full) {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (j0 + 16 * (e >> 2) + 4 * grp + (e & 3) >= np) x[e] = -INFINITY;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) mt = fmaxf(mt, x[e]);
      mt = fmaxf(mt, lane_xor(mt, 16));
      mt = fmaxf(mt, lane_xor(mt, 32));
      const float mn = fmaxf(m_run, mt);
      const bool need = mn > m_run + kRescaleThreshold;
      const bool rescale = __any(need);
      float alpha = 1.f;
      if (rescale) {
        alpha = need ? fast_exp2(m_run - mn) : 1.f;
        if (need) m_run = mn;
        l_run *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      uint32_t pw[4];
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fast_exp2(x[e] - m_use);
        const float p1 = fast_exp2(x[e + 1] - m_use);
        const uint32_t pk = pack_bf16x2(p0, p1);
        lsum += bf16lo(pk) + bf16hi(pk);
        pw[e >> 1] = pk;
      }
      l_run += lsum;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      if (rescale) {
        // rare (the running maximum rose by more than 8): a real branch - the
        // asm keeps the compiler from turning it into selects executed on every
        // tile, which would also pull the accumulators out of their registers
        asm volatile("" ::: "memory");
#pragma unroll
        for (int blk = 0; blk < DBLK; ++blk) oacc[blk] *= alpha;
      }
      // O^T += V^T P^T, fragments read PVD MFMAs ahead
#pragma unroll
      for (int blk = 0; blk < DBLK; ++blk) {
        const bf16x8 va = vf[blk % PVD];
        if (blk + PVD < DBLK) vf[blk % PVD] = vread(blk + PVD);
        oacc[blk] = mfma16x16x32(va, pb, oacc[blk]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (blk + PVD < DBLK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };
  // super-iteration u: wait for this wavefront's fetches of super-stage ss,
  // barrier, start the fetches of super-iteration u + NSUP - 1 (into the
  // super-stage u - 1 used), compute tile u of this key half
  const int n_sup = KS == 1 ? n_live : max(n_h0, n_h1);
  const int n_mine = kh == 0 ? n_h0 : n_h1;
  auto step = [&](const int u, const int ss) __attribute__((always_inline)) {
    wait_vmcnt<KS * PW * (NSUP - 2)>();
    tile_barrier();
    int jn[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) jn[k] = key_of(k, u + NSUP - 1);
    const int ssn = (ss + NSUP - 1) % NSUP;
    fetch_group(0, jn, ssn);
    if (KS == 1 || u < n_mine) {
      tile_step(key_of(kh, u), ss, jn, ssn);
    } else {
      // no tile for this key half: the fetches still go out
#pragma unroll
      for (int g = 1; g < kFG; ++g) fetch_group(g, jn, ssn);
    }
  };
  if constexpr (NSUP == 2) {
    // two super-stages per iteration: each known at compile time
    for (int u = 0; u < n_sup; u += 2) {
      step(u, 0);
      if (u + 1 < n_sup) step(u + 1, 1);
    }
  } else {
    for (int u = 0; u < n_sup; ++u) step(u, u % NSUP);
  }
  // the fetches of the re-fetched tail stages must land before the workgroup
  // (and its LDS) ends
  wait_vmcnt<0>();
  if constexpr (kAsmAcc) acc_settle(oacc);
  // KS = 2: half 1 leaves (m, l, O^T) in the first XO_BYTES of the stage area;
  // the output rows are staged after it
  constexpr int NACC = DBLK * (RW == 32 ? 16 : 4);
  constexpr int NF = NACC + 2;
  constexpr int XO_BYTES = KS == 2 ? NWR * NF * 64 * 4 : 0;
  if constexpr (KS == 2) {
    // merge the key halves: half 1 leaves (m, l, O^T) in LDS (the stages are
    // free now), half 0 rescales both to the larger maximum and adds
    float* xo = reinterpret_cast<float*>(stages) + (size_t)rg * NF * 64 + lane;
    __syncthreads();
    if (kh == 1) {
      xo[0] = m_run;
      xo[64] = l_run;
#pragma unroll
      for (int blk = 0; blk < DBLK; ++blk)
#pragma unroll
        for (int e = 0; e < NACC / DBLK; ++e) xo[(2 + blk * (NACC / DBLK) + e) * 64] = oacc[blk][e];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = xo[0], l1 = xo[64];
    const float mm = fmaxf(m_run, m1);
    const float f0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mm);
    const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
    l_run = l_run * f0 + l1 * f1;
#pragma unroll
    for (int blk = 0; blk < DBLK; ++blk)
#pragma unroll
      for (int e = 0; e < NACC / DBLK; ++e)
        oacc[blk][e] = oacc[blk][e] * f0 + xo[(2 + blk * (NACC / DBLK) + e) * 64] * f1;
  } else {
    // every wavefront is done with the stages (and every fetch has landed)
    // before any of them is overwritten by the output rows below
    __syncthreads();
  }

  // ---- 5. normalise, stage the rows in LDS, store whole rows -----------------
  // O^T holds one query row per lane column, so stored straight from the
  // registers each instruction would write 8-byte pieces of RW different rows
  // (measured: the long prefill's 128 MB of output at 1.6 TB/s). The wavefront
  // writes its normalised bf16 rows into its own part of the stage area
  // instead (16-byte chunk c of row r at c ^ (r & 15): rows 1 KB apart fall on
  // different banks) and stores them back row by row: each store instruction
  // writes 64 consecutive 16-byte chunks of the output. Where the stage area
  // cannot hold every wavefront's whole rows, the columns go in NPASS passes.
  float l_tot = l_run;
  if constexpr (RW == 16) l_tot += lane_xor(l_tot, 16);
  l_tot += lane_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int NPASS = XO_BYTES + NWR * RW * DV * 2 <= NSTAGE * STAGE_BYTES ? 1 : 2;
  constexpr int DVP = DV / NPASS;                      // columns per pass
  static_assert(XO_BYTES + NWR * RW * DVP * 2 <= NSTAGE * STAGE_BYTES, "output staging area");
  constexpr int CPRO = DVP / 8;                        // 16-byte chunks per staged row
  constexpr int OSWZ = CPRO >= 16 ? 15 : CPRO - 1;
  constexpr int RPO = 64 / CPRO;                       // rows per store instruction
  static_assert(64 % CPRO == 0 && RW % RPO == 0 && DBLK % NPASS == 0, "output rows per store");
  const unsigned ost = (lds_addr(stages) + (unsigned)(XO_BYTES + rg * RW * DVP * 2)) & kLdsMask;
  auto ost_at = [&](int r, int c) { return (unsigned)(r * DVP * 2 + 16 * (c ^ (r & OSWZ))); };
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    constexpr int BPP = DBLK / NPASS;                  // d blocks per pass
    if constexpr (RW == 32) {
      // O^T lane l: row l % 32, d = 32*blk + 8*i + 4*(l/32) + jj: chunk 4*blk + i
      // of the pass, bytes 8*(l/32) .. +7
#pragma unroll
      for (int bb = 0; bb < BPP; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int blk = pass * BPP + bb;
          u32x2 pk;
          pk.x = pack_bf16x2(oacc[blk][4 * i + 0] * inv, oacc[blk][4 * i + 1] * inv);
          pk.y = pack_bf16x2(oacc[blk][4 * i + 2] * inv, oacc[blk][4 * i + 3] * inv);
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
              (size_t)(ost + ost_at(col, 4 * bb + i) + 8 * grp)) = pk;
        }
    } else {
      // O^T lane l: row l % 16, d = 16*blk + 4*(l/16) + e: chunk 2*blk + (l/16)/2
      // of the pass, bytes 8*((l/16) % 2) .. +7
#pragma unroll
      for (int bb = 0; bb < BPP; ++bb) {
        const int blk = pass * BPP + bb;
        u32x2 pk;
        pk.x = pack_bf16x2(oacc[blk][0] * inv, oacc[blk][1] * inv);
        pk.y = pack_bf16x2(oacc[blk][2] * inv, oacc[blk][3] * inv);
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
            (size_t)(ost + ost_at(col, 2 * bb + (grp >> 1)) + 8 * (grp & 1))) = pk;
      }
    }
    // back row by row (this wavefront's own LDS: no barrier; the compiler
    // waits for the writes before the reads, and LDS accesses of one
    // wavefront take effect in order, so the next pass overwrites only what
    // was read), with non-temporal stores: the output is not read again here,
    // and the caches keep the K/V tiles other workgroups still fetch (vision
    // chunk 41.9 -> 40.6 us, long prefill 349.9 -> 343.4 us)
#pragma unroll
    for (int k = 0; k < RW / RPO; ++k) {
      const int rl = k * RPO + lane / CPRO, c = lane % CPRO;
      const u32x4 v = lds_at<u32x4>(ost, ost_at(rl, c));
      const int rr = RW * rg + rl;   // the workgroup's row: token rr / G of the tile, head rr % G
      const int so = s0 + rr / G;
      if (rr < MQ * G && so < p.S_q)
        st_stream<u32x4>((uint16_t*)p.out + ((b * p.Hq + hk * G + rr % G) * p.S_q + so) * (int64_t)DV +
                             pass * DVP + 8 * c, v);
    }
  }
}

namespace {

// Live-tile map of the bias variant: bit kt % 32 of word (b, qt, kt / 32) is
// set iff some row of query tile qt (MQ tokens from qt * MQ) allows some key
// of key tile kt below nonpad (a bias entry other than -inf) - the set a
// workgroup's own bias scan finds (build_live_list), computed once per batch
// row instead of once per KV head, by a grid that keeps the memory busy.
// One workgroup per (b, query tile, byte of a word = 8 key tiles = 256 keys),
// which writes its byte of the word; a byte wholly at or past nonpad is
// written 0 without loads. Small workgroups keep many of them in flight on
// every CU, so the pass costs about one memory round trip. The byte is the
// slowest index of the grid: consecutive workgroups are dealt round-robin over
// the XCDs, and with the byte fastest every workgroup of a low word (the ones
// below nonpad, which do the loads) could land on the same few XCDs, leaving
// the others idle.
constexpr int kMapTilesPerGroup = 8;
template <typename BiasT>
__global__ __launch_bounds__(256) void tilemap_kernel(const BiasT* __restrict__ bias,
                                                      const int64_t* __restrict__ nonpad,
                                                      uint32_t* __restrict__ map, int S_q, int T,
                                                      int MQ, int n_qt, int n_words) {
  constexpr int GPW = 32 / kMapTilesPerGroup;    // workgroups (bytes) per word
  __shared__ uint32_t s_bits;
  const int n_bq = gridDim.x / (n_words * GPW);  // (b, query tile) pairs
  const int unit = blockIdx.x / n_bq;            // word * GPW + byte
  const int qt = (blockIdx.x % n_bq) % n_qt;
  const int64_t b = (blockIdx.x % n_bq) / n_qt;
  const int wid = (int)(b * n_qt + qt) * n_words + unit / GPW;   // the map's layout: [b][query tile][word]
  uint8_t* const out = reinterpret_cast<uint8_t*>(map + wid) + unit % GPW;
  const int np = (int)clamp_nonpad(nonpad[b], T);
  const int s0 = qt * MQ, nrows = min(MQ, S_q - s0);
  const int j_lo = unit * kMapTilesPerGroup * kTileKeys, j_hi = min(j_lo + kMapTilesPerGroup * kTileKeys, np);
  if (j_lo >= np || nrows <= 0) {
    if (threadIdx.x == 0) *out = 0;
    return;
  }
  if (threadIdx.x == 0) s_bits = 0u;
  __syncthreads();
  constexpr int EPV = 16 / (int)sizeof(BiasT);
  constexpr int CPW = kMapTilesPerGroup * kTileKeys / EPV;   // 16-byte chunks of a row's 256 keys
  constexpr int RPP = 256 / CPW;                             // rows per pass
  const int c = threadIdx.x % CPW, rr = threadIdx.x / CPW;
  const int j = j_lo + c * EPV;               // rows are multiples of 16 bytes
  bool any = false;
  if (j < j_hi) {
    const BiasT* col = bias + ((int64_t)b * S_q + s0) * T + j;
    constexpr int U = 8;  // loads in flight per thread (rows past the tile repeat its last)
    for (int r0 = rr; r0 < nrows; r0 += U * RPP) {
      u32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = ld_global<u32x4>(col + (int64_t)min(r0 + u * RPP, nrows - 1) * T);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        BiasT vals[EPV];
        *reinterpret_cast<u32x4*>(vals) = raw[u];
#pragma unroll
        for (int e = 0; e < EPV; ++e) any |= (j + e < np) && live_bits<BiasT>(vals[e]);
      }
    }
  }
  // OR the lanes' tile bits over the wavefront: one LDS atomic per wavefront
  // instead of one per lane on the same word
  const unsigned bits = wave_or_u32(any ? 1u << ((c * EPV) / kTileKeys) : 0u);
  if ((threadIdx.x & 63) == 0 && bits) atomicOr(&s_bits, bits);
  __syncthreads();
  if (threadIdx.x == 0) *out = (uint8_t)s_bits;
}

template <int D, int RW, int NW, bool kRules, typename BiasT, bool kQReg, int KS, int DV>
hipError_t launch_dma_inst(const AttnParams& p, hipStream_t stream) {
  using Geo = DmaGeom<D, RW, NW, kRules, BiasT, kQReg, KS, DV>;
  const int MQ = (RW * NW / KS) / p.G;
  const int n_qt = (p.S_q + MQ - 1) / MQ;
  const int n_kt = num_tiles(p.T);
  const size_t list = (size_t)((n_kt + 31) / 32) * 4 + (size_t)n_kt * 2;
  const size_t lds = (size_t)Geo::Q_BYTES + (size_t)Geo::NSTAGE * Geo::STAGE_BYTES +
                     ((list + 15) & ~(size_t)15);
  auto kern = attn_prefill_dma_kernel<D, RW, NW, kRules, BiasT, kQReg, KS, DV>;
  // opt in to exactly the dynamic LDS of this launch (the kernel's static LDS
  // comes on top)
  {
    const hipError_t e = opt_in_dynamic_lds((const void*)kern, lds);
    if (e != hipSuccess) {
      set_launch_detail("hipFuncSetAttribute(MaxDynamicSharedMemorySize), direct-to-LDS prefill");
      return e;
    }
  }
  AttnParams pp = p;
  pp.tilemap = nullptr;
  if constexpr (!kRules) {
    // the live-tile map, when the caller's scratch holds it
    const int n_words = (n_kt + 31) / 32;
    const size_t need = (size_t)p.B * n_qt * n_words * sizeof(uint32_t);
    const int64_t map_groups = (int64_t)p.B * n_qt * n_words * (32 / kMapTilesPerGroup);
    // (a launch covers fewer than 2^32 work-items; past that the workgroups
    // scan their bias rows themselves)
    if (p.ws != nullptr && p.ws_bytes >= need && map_groups * 256 <= (int64_t)UINT32_MAX) {
      hipLaunchKernelGGL(tilemap_kernel<BiasT>, dim3((unsigned)map_groups), dim3(256),
                         0, stream, (const BiasT*)p.bias, p.nonpad, (uint32_t*)p.ws, p.S_q, p.T, MQ, n_qt,
                         n_words);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) {
        set_launch_detail("live-tile map kernel launch");
        return e;
      }
      pp.tilemap = (const uint32_t*)p.ws;
    }
  }
  const dim3 grid((unsigned)((int64_t)n_qt * p.B * p.Hkv));
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, stream, pp, n_qt);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) set_launch_detail("direct-to-LDS prefill kernel launch");
  return e;
}

// kQReg: Q^T fragments in registers (RW = 16 always; RW = 32 where the
// accumulators live in the accumulation registers)
// KS = 2: two wavefronts per row group, on alternate tiles
// DV: the V head size (that of the output rows)
template <int D, int RW, int NW, bool kQReg = (RW == 16), int KS = 1, int DV = D>
hipError_t launch_dma_v(const AttnParams& p, hipStream_t stream) {
  if (p.bias == nullptr) return launch_dma_inst<D, RW, NW, true, uint16_t, kQReg, KS, DV>(p, stream);
  if (p.bias_is_bf16) return launch_dma_inst<D, RW, NW, false, uint16_t, kQReg, KS, DV>(p, stream);
  return launch_dma_inst<D, RW, NW, false, uint32_t, kQReg, KS, DV>(p, stream);
}

}  // namespace

}  // namespace abgqa
