// bf16 prefill attention over the static cache on the gfx950 matrix cores.
//
// What it computes: onnxruntime skill "cuda-attention-kernel-patterns",
// section 4 (scale * QK^T, + bias, softmax, times V), section 6 (rows with no
// allowed key write zeros; masked keys removed by selection), section 11
// (external cache: keys are the slots < nonpad_kv_seqlen); mobius issue #366
// (the float bias carries causal, window, block-overlay and padding rules);
// query head h reads KV head h / G (onnxruntime PR #28242, CPU GQA excerpt).
// Prefill is where a fused tiled kernel pays (mobius skill
// "attention-optimization", "Flash Attention: when it actually helps").
//
// Layout of the work
//   workgroup  one (b, kv head, query tile): NW wavefronts of 32 rows each,
//              r = s_local * G + g, i.e. MQ = 32*NW / G consecutive query
//              tokens times the G heads of the group. Every K/V tile staged
//              in LDS is read by all G heads' rows.
//   tiles      32 keys. The workgroup first lists its live tiles: tiles below
//              nonpad that hold an allowed entry for one of its rows (scanned
//              from the bias, or derived from the rules). Skipping is exact:
//              a masked key contributes exactly zero.
//   LDS        per tile, K and V row-major [32][D] bf16, 16-byte chunks XOR-
//              swizzled by swz_bits<D>(row) against bank conflicts; double-buffered.
//   S^T = K Q^T    32x32x16 bf16 MFMA: A = K rows from LDS, B = Q^T held in
//                  registers for the whole loop. Result lane l: query row
//                  (l % 32), keys 8*i + 4*(l/32) + j (i, j < 4).
//   softmax        a row's 32 scores sit in lanes l and l^32 (16 each); base 2;
//                  weights rounded to bf16 (RNE), the row sum adds the rounded
//                  weights; the running max moves only when exceeded by > 8.
//   O^T += V^T P^T 32x32x16 MFMA per (32-d block, 16-key step): B = P^T is 8
//                  consecutive score registers, A = V^T comes from two
//                  transposing LDS reads (ds_read_b64_tr_b16) of the row-major
//                  V tile. O^T lane l: query row l % 32, d = 32*blk + 8*i +
//                  4*(l/32) + j.
// The next tile's bias values (registers) and K/V (registers, then LDS) are
// fetched while the current tile is computed; the bias loads are issued first
// so that waiting for them never waits for the K/V loads behind them.
#include <stdlib.h>

#include "prefill_common.h"

namespace abgqa {

namespace {

// 4 consecutive bias values of one row, packed (bf16: 2 words, fp32: 4 words)
template <typename BiasT> struct Bias4;
template <> struct Bias4<uint16_t> {
  u32x2 w;
  __device__ __forceinline__ uint16_t get(int e) const {
    const uint32_t x = (e < 2) ? w.x : w.y;
    return (e & 1) ? (uint16_t)(x >> 16) : (uint16_t)(x & 0xffff);
  }
};
template <> struct Bias4<uint32_t> {
  u32x4 w;
  __device__ __forceinline__ uint32_t get(int e) const { return w[e]; }
};

// keys j..j+3 of a bias row; `vec` (uniform): rows are 4-aligned, so one
// aligned load at min(j, T-4); else element loads clamped into the row.
// Values for keys past the row end are never used (those keys are masked).
__device__ __forceinline__ Bias4<uint16_t> load_bias4(const uint16_t* row, int j, int T, bool vec) {
  Bias4<uint16_t> b;
  if (vec) {
    b.w = ld_global<u32x2>(row + min(j, T - 4));
  } else {
    const uint32_t e0 = row[min(j, T - 1)], e1 = row[min(j + 1, T - 1)];
    const uint32_t e2 = row[min(j + 2, T - 1)], e3 = row[min(j + 3, T - 1)];
    b.w = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
  }
  return b;
}
__device__ __forceinline__ Bias4<uint32_t> load_bias4(const uint32_t* row, int j, int T, bool vec) {
  Bias4<uint32_t> b;
  if (vec) {
    b.w = ld_global<u32x4>(row + min(j, T - 4));
  } else {
    b.w = u32x4{row[min(j, T - 1)], row[min(j + 1, T - 1)], row[min(j + 2, T - 1)],
                row[min(j + 3, T - 1)]};
  }
  return b;
}

}  // namespace

size_t prefill_lds_bytes(int D, int max_seq) {
  const int nt = num_tiles(max_seq);
  const size_t words = (size_t)((nt + 31) / 32) * 4;  // live bitmap
  const size_t list = (size_t)nt * 2;                 // live tile list (u16)
  const size_t stage = (size_t)2 * kTileKeys * D * 2;  // K and V
  return 2 * stage + ((words + list + 15) & ~(size_t)15);
}



template <int D, int NW, bool kRules, typename BiasT>
__global__ __launch_bounds__(NW * 64) void attn_prefill_kernel(AttnParams p, int n_qt) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;              // k-steps of S^T over the head dim
  constexpr int DBLK = D / 32;                // 32-wide d blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int CH = kTileKeys * CPR;         // chunks per K (or V) tile
  constexpr int CPT = (CH + NT - 1) / NT;     // chunks per thread per tensor
  constexpr int TILE_ELEMS = kTileKeys * D;
  constexpr int STAGE_ELEMS = 2 * TILE_ELEMS;

  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* stages = reinterpret_cast<__bf16*>(smem);
  const int T = p.T, G = p.G;
  const int n_kt_max = num_tiles(T);
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(smem + (size_t)2 * STAGE_ELEMS * 2);
  const int n_words = (n_kt_max + 31) / 32;
  uint16_t* s_list = reinterpret_cast<uint16_t*>(s_bits + n_words);
  __shared__ int s_nlive;
  __shared__ int32_t s_ids[4];
  __shared__ int s_nids;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;   // query row within the wavefront
  const int hh = lane >> 5;    // half of the wavefront

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = n_qt - 1 - (wg % n_qt);   // later (heavier) query tiles first
  const int bh = wg / n_qt;
  const int hk = bh % p.Hkv;
  const int64_t b = bh / p.Hkv;
  const int np = (int)clamp_nonpad(p.nonpad[b], T);
  const int MQ = (32 * NW) / G;
  const int s0 = qt * MQ;
  const int s_end = min(s0 + MQ, p.S_q);
  const int n_kt = num_tiles(np);

  // ---- 1. live tiles ---------------------------------------------------------
  const int n_live = build_live_list<NT, kRules, BiasT>(p, b, np, s0, s_end, n_kt, s_bits, s_list,
                                                       n_words, s_ids, &s_nids, &s_nlive);

  // ---- 2. this lane's query row and its Q^T fragments ------------------------
  const int r = 32 * w + col;
  const int sl = r / G, g = r % G;
  const int s = s0 + sl;
  const bool row_ok = (r < MQ * G) && (s < p.S_q);
  const int h = hk * G + g;
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qp = (const __bf16*)p.q + ((b * p.Hq + h) * p.S_q + (row_ok ? s : 0)) * (int64_t)D + 8 * hh;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) qf[i] = row_ok ? ld_global<bf16x8>(qp + 16 * i) : bf16x8{};
  }
  RowRule rule{};
  if constexpr (kRules) {
    if (row_ok) rule = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window, p.circular);
  }
  const BiasT* brow = kRules ? nullptr : (const BiasT*)p.bias + (b * p.S_q + (row_ok ? s : 0)) * (int64_t)T;
  const int32_t* kindb = p.slot_kind ? p.slot_kind + b * T : nullptr;
  const bool vec4 = (T % 4) == 0;   // bias / kind rows 4-aligned (uniform)
  const float scale_log2 = p.scale * kLog2e;
  const bool cap_on = p.softcap > 0.f;
  const float cap2 = p.softcap * kLog2e, scale_over_cap = cap_on ? p.scale / p.softcap : 0.f;

  const __bf16* kg = (const __bf16*)p.k + (b * p.Hkv + hk) * (int64_t)T * D;
  const __bf16* vg = (const __bf16*)p.v + (b * p.Hkv + hk) * (int64_t)T * D;

  // ---- 3. staging: bias/kinds -> registers; K/V -> registers -> LDS ----------
  struct TileMask {
    Bias4<BiasT> bias[4];
    int4 kind[4];
  };
  // this lane's 16 keys of tile t: j0 + 8*i + 4*hh + (0..3)
  auto mask_load = [&](int t, TileMask& m) {
    const int j0 = (int)s_list[t] * kTileKeys;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jb = j0 + 8 * i + 4 * hh;
      if constexpr (kRules) {
        int4 k4 = {0, 0, 0, 0};
        if (kindb) {
          if (vec4) {
            k4 = ld_global<int4>(kindb + min(jb, T - 4));
          } else {
            k4.x = kindb[min(jb, T - 1)]; k4.y = kindb[min(jb + 1, T - 1)];
            k4.z = kindb[min(jb + 2, T - 1)]; k4.w = kindb[min(jb + 3, T - 1)];
          }
        }
        m.kind[i] = k4;
      } else {
        m.bias[i] = load_bias4(brow, jb, T, vec4);
      }
    }
  };
  // K and V of a tile move global -> registers -> LDS. At D = 512 the two go
  // through one register buffer in turn (K during S^T, V during PV): Q^T and
  // the O^T accumulators leave no room for both.
  constexpr bool kTwoPhase = D >= 512;
  bf16x8 kreg[CPT];
  bf16x8 vreg[kTwoPhase ? 1 : CPT];
  auto load_rows = [&](int t, const __bf16* src, bf16x8* dst) {
    const int j0 = (int)s_list[t] * kTileKeys;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = min(tid + i * NT, CH - 1);
      const int kk = c / CPR, dc = c % CPR;
      const int j = min(j0 + kk, np - 1);   // clamped: rows past nonpad are zeroed below
      dst[i] = ld_global<bf16x8>(src + (int64_t)j * D + 8 * dc);
    }
  };
  auto store_rows = [&](int t, __bf16* tile, const bf16x8* src) {
    const int j0 = (int)s_list[t] * kTileKeys;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CH % NT == 0 || c < CH) {
        const int kk = c / CPR, dc = c % CPR;
        // keys past nonpad hold arbitrary bits: select zeros (never multiply them)
        *reinterpret_cast<bf16x8*>(tile + swz<D>(kk, dc)) = (j0 + kk < np) ? src[i] : bf16x8{};
      }
    }
  };
  auto stage_load = [&](int t) {
    load_rows(t, kg, kreg);
    if constexpr (!kTwoPhase) load_rows(t, vg, vreg);
  };
  auto stage_store = [&](int t, int buf) {
    __bf16* ks = stages + buf * STAGE_ELEMS;
    store_rows(t, ks, kreg);
    if constexpr (!kTwoPhase) store_rows(t, ks + TILE_ELEMS, vreg);
  };

  // ---- 4. main loop ---------------------------------------------------------
  f32x16 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // tr16 addressing of V^T: lane L = 16*gq + 4*kq + jq reads
  // V[16*step + 8*half + 4*(gq/2) + kq][32*blk + 16*(gq%2) + 4*jq]
  const int gq = lane >> 4, kq = (lane >> 2) & 3, jq = lane & 3;
  const int vkey0 = 4 * (gq >> 1) + kq;
  const int vdofs = 16 * (gq & 1) + 4 * jq;

  TileMask mcur, mnxt;
  if (n_live > 0) {
    mask_load(0, mcur);
    stage_load(0);
    stage_store(0, 0);
    if constexpr (kTwoPhase) {
      load_rows(0, vg, kreg);
      store_rows(0, stages + TILE_ELEMS, kreg);
    }
  }
  __syncthreads();
  for (int t = 0; t < n_live; ++t) {
    const int buf = t & 1;
    const int j0 = (int)s_list[t] * kTileKeys;
    const bool more = t + 1 < n_live;
    if (more) {
      mask_load(t + 1, mnxt);   // small loads first (see the header)
      stage_load(t + 1);
    }

    // S^T = K Q^T
    const __bf16* ks = stages + buf * STAGE_ELEMS;
    const __bf16* vs = ks + TILE_ELEMS;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + swz<D>(col, 2 * i + hh));
      sacc = mfma32x32x16(a, qf[i], sacc);
    }

    // softcap (0 = none) on scale * q.k, before the bias
    float sl = scale_log2;
    if (cap_on) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = softcap_base2(sacc[e], cap2, scale_over_cap);
      sl = 1.f;
    }
    // keep = valid && allowed; x = keep ? (s*scale + bias)*log2e : -inf
    float x[16];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = j0 + 8 * i + 4 * hh + jj;
        bool keep;
        float badd = 0.f;
        if constexpr (kRules) {
          const int kj = jj == 0 ? mcur.kind[i].x : jj == 1 ? mcur.kind[i].y
                       : jj == 2 ? mcur.kind[i].z : mcur.kind[i].w;
          keep = row_ok & (j < np) & rule.allowed(j, kj);
        } else {
          const BiasT bv = mcur.bias[i].get(jj);
          keep = row_ok & (j < np) & live_bits<BiasT>(bv);
          badd = bias_f32<BiasT>(bv) * kLog2e;
        }
        const float v = fmaf(sacc[4 * i + jj], sl, badd);
        x[4 * i + jj] = keep ? v : -INFINITY;
        mt = fmaxf(mt, x[4 * i + jj]);
      }
    mt = fmaxf(mt, lane_xor(mt, 32));
    const float mn = fmaxf(m_run, mt);
    const bool need = mn > m_run + kRescaleThreshold;
    const bool rescale = __any(need);   // wave-uniform
    float alpha = 1.f;
    if (rescale) {
      alpha = need ? fast_exp2(m_run - mn) : 1.f;
      if (need) m_run = mn;
      l_run *= alpha;
    }
    // weights, rounded to bf16; P^T for the two 16-key steps
    uint32_t pw[8];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = (x[e] == -INFINITY) ? 0.f : fast_exp2(x[e] - m_run);
      const float p1 = (x[e + 1] == -INFINITY) ? 0.f : fast_exp2(x[e + 1] - m_run);
      const uint32_t pk = pack_bf16x2(p0, p1);
      lsum += bf16lo(pk) + bf16hi(pk);
      pw[e >> 1] = pk;
    }
    l_run += lsum;
    const bf16x8 pb0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    const bf16x8 pb1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
    if constexpr (kTwoPhase) {
      if (more) {   // K of the next tile to LDS, then its V into the same registers
        store_rows(t + 1, stages + (buf ^ 1) * STAGE_ELEMS, kreg);
        load_rows(t + 1, vg, kreg);
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int blk = 0; blk < DBLK; ++blk) {
      // the O^T rescale, one 32-d block at a time right before its MFMAs, keeps
      // only 16 accumulators in flight through the vector registers
      if (rescale) oacc[blk] *= alpha;
      const int d = 32 * blk + vdofs;
      const int c = d >> 3, within = d & 7;
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const int k0 = 16 * step + vkey0;
        const u32x2 lo = lds_read_tr16(vs + swz<D>(k0, c) + within);
        const u32x2 hi = lds_read_tr16(vs + swz<D>(k0 + 8, c) + within);
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        oacc[blk] = mfma32x32x16(va, step == 0 ? pb0 : pb1, oacc[blk]);
      }
    }

    if (more) {
      if constexpr (kTwoPhase) store_rows(t + 1, stages + (buf ^ 1) * STAGE_ELEMS + TILE_ELEMS, kreg);
      else stage_store(t + 1, buf ^ 1);
      mcur = mnxt;
    }
    __syncthreads();
  }

  // ---- 5. normalise and store -----------------------------------------------
  const float l_tot = l_run + lane_xor(l_run, 32);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = (uint16_t*)p.out + ((b * p.Hq + h) * p.S_q + s) * (int64_t)D + 4 * hh;
#pragma unroll
    for (int blk = 0; blk < DBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 pk;
        pk.x = pack_bf16x2(oacc[blk][4 * i + 0] * inv, oacc[blk][4 * i + 1] * inv);
        pk.y = pack_bf16x2(oacc[blk][4 * i + 2] * inv, oacc[blk][4 * i + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * blk + 8 * i) = pk;
      }
  }
}

// The same computation with 16-row wavefronts (16x16x32 MFMAs), for D = 512:
// a 32-row wavefront would need 256 accumulator registers for O^T at D = 512
// plus 128 for Q^T, more than one lane has. Rows r = 16*w + (lane % 16);
// S^T lane l: query row l % 16, keys 16*kb + 4*(l/16) + e; O^T lane l: query
// row l % 16, d = 16*blk + 4*(l/16) + e. V^T comes from two transposing reads
// per (16-d block): lane 16*g + 4*k + j addresses V[4*g + k (+16)][16*blk + 4*j].
template <int D, int NW, bool kRules, typename BiasT>
__global__ __launch_bounds__(NW * 64) void attn_prefill16_kernel(AttnParams p, int n_qt) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 32;
  constexpr int DBLK = D / 16;
  constexpr int CPR = D / 8;
  constexpr int CH = kTileKeys * CPR;
  constexpr int CPT = (CH + NT - 1) / NT;
  constexpr int TILE_ELEMS = kTileKeys * D;
  constexpr int STAGE_ELEMS = 2 * TILE_ELEMS;

  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* stages = reinterpret_cast<__bf16*>(smem);
  const int T = p.T, G = p.G;
  const int n_kt_max = num_tiles(T);
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(smem + (size_t)2 * STAGE_ELEMS * 2);
  const int n_words = (n_kt_max + 31) / 32;
  uint16_t* s_list = reinterpret_cast<uint16_t*>(s_bits + n_words);
  __shared__ int s_nlive;
  __shared__ int32_t s_ids[4];
  __shared__ int s_nids;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;   // query row within the wavefront
  const int grp = lane >> 4;   // k-slot group

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = n_qt - 1 - (wg % n_qt);
  const int bh = wg / n_qt;
  const int hk = bh % p.Hkv;
  const int64_t b = bh / p.Hkv;
  const int np = (int)clamp_nonpad(p.nonpad[b], T);
  const int MQ = (16 * NW) / G;
  const int s0 = qt * MQ;
  const int s_end = min(s0 + MQ, p.S_q);
  const int n_kt = num_tiles(np);

  const int n_live = build_live_list<NT, kRules, BiasT>(p, b, np, s0, s_end, n_kt, s_bits, s_list,
                                                       n_words, s_ids, &s_nids, &s_nlive);

  const int r = 16 * w + col;
  const int sl = r / G, g = r % G;
  const int s = s0 + sl;
  const bool row_ok = (r < MQ * G) && (s < p.S_q);
  const int h = hk * G + g;
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qp = (const __bf16*)p.q + ((b * p.Hq + h) * p.S_q + (row_ok ? s : 0)) * (int64_t)D + 8 * grp;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) qf[i] = row_ok ? ld_global<bf16x8>(qp + 32 * i) : bf16x8{};
  }
  RowRule rule{};
  if constexpr (kRules) {
    if (row_ok) rule = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window, p.circular);
  }
  const BiasT* brow = kRules ? nullptr : (const BiasT*)p.bias + (b * p.S_q + (row_ok ? s : 0)) * (int64_t)T;
  const int32_t* kindb = p.slot_kind ? p.slot_kind + b * T : nullptr;
  const bool vec4 = (T % 4) == 0;
  const float scale_log2 = p.scale * kLog2e;
  const bool cap_on = p.softcap > 0.f;
  const float cap2 = p.softcap * kLog2e, scale_over_cap = cap_on ? p.scale / p.softcap : 0.f;
  const __bf16* kg = (const __bf16*)p.k + (b * p.Hkv + hk) * (int64_t)T * D;
  const __bf16* vg = (const __bf16*)p.v + (b * p.Hkv + hk) * (int64_t)T * D;

  struct TileMask {
    Bias4<BiasT> bias[2];
    int4 kind[2];
  };
  // this lane's 8 keys of tile t: j0 + 16*kb + 4*grp + (0..3)
  auto mask_load = [&](int t, TileMask& m) {
    const int j0 = (int)s_list[t] * kTileKeys;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int jb = j0 + 16 * kb + 4 * grp;
      if constexpr (kRules) {
        int4 k4 = {0, 0, 0, 0};
        if (kindb) {
          if (vec4) {
            k4 = ld_global<int4>(kindb + min(jb, T - 4));
          } else {
            k4.x = kindb[min(jb, T - 1)]; k4.y = kindb[min(jb + 1, T - 1)];
            k4.z = kindb[min(jb + 2, T - 1)]; k4.w = kindb[min(jb + 3, T - 1)];
          }
        }
        m.kind[kb] = k4;
      } else {
        m.bias[kb] = load_bias4(brow, jb, T, vec4);
      }
    }
  };
  bf16x8 kreg[CPT], vreg[CPT];
  auto stage_load = [&](int t) {
    const int j0 = (int)s_list[t] * kTileKeys;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = min(tid + i * NT, CH - 1);
      const int kk = c / CPR, dc = c % CPR;
      const int j = min(j0 + kk, np - 1);
      kreg[i] = ld_global<bf16x8>(kg + (int64_t)j * D + 8 * dc);
      vreg[i] = ld_global<bf16x8>(vg + (int64_t)j * D + 8 * dc);
    }
  };
  auto stage_store = [&](int t, int buf) {
    const int j0 = (int)s_list[t] * kTileKeys;
    __bf16* ks = stages + buf * STAGE_ELEMS;
    __bf16* vs = ks + TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (CH % NT == 0 || c < CH) {
        const int kk = c / CPR, dc = c % CPR;
        const bool ok = j0 + kk < np;   // keys past nonpad: zeros, never their bits
        *reinterpret_cast<bf16x8*>(ks + swz<D>(kk, dc)) = ok ? kreg[i] : bf16x8{};
        *reinterpret_cast<bf16x8*>(vs + swz<D>(kk, dc)) = ok ? vreg[i] : bf16x8{};
      }
    }
  };

  f32x4 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int vkey0 = lane >> 2;          // 4*g + k for lane 16*g + 4*k + j
  const int vdofs = 4 * (lane & 3);     // 4*j

  TileMask mcur, mnxt;
  if (n_live > 0) {
    mask_load(0, mcur);
    stage_load(0);
    stage_store(0, 0);
  }
  __syncthreads();
  for (int t = 0; t < n_live; ++t) {
    const int buf = t & 1;
    const int j0 = (int)s_list[t] * kTileKeys;
    const bool more = t + 1 < n_live;
    if (more) {
      mask_load(t + 1, mnxt);
      stage_load(t + 1);
    }
    const __bf16* ks = stages + buf * STAGE_ELEMS;
    const __bf16* vs = ks + TILE_ELEMS;
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + swz<D>(16 * kb + col, 4 * i + grp));
        sacc[kb] = mfma16x16x32(a, qf[i], sacc[kb]);
      }
    }
    float sl = scale_log2;
    if (cap_on) {   // softcap (0 = none) on scale * q.k, before the bias
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[kb][e] = softcap_base2(sacc[kb][e], cap2, scale_over_cap);
      sl = 1.f;
    }
    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 16 * kb + 4 * grp + e;
        bool keep;
        float badd = 0.f;
        if constexpr (kRules) {
          const int kj = e == 0 ? mcur.kind[kb].x : e == 1 ? mcur.kind[kb].y
                       : e == 2 ? mcur.kind[kb].z : mcur.kind[kb].w;
          keep = row_ok & (j < np) & rule.allowed(j, kj);
        } else {
          const BiasT bv = mcur.bias[kb].get(e);
          keep = row_ok & (j < np) & live_bits<BiasT>(bv);
          badd = bias_f32<BiasT>(bv) * kLog2e;
        }
        const float v = fmaf(sacc[kb][e], sl, badd);
        x[4 * kb + e] = keep ? v : -INFINITY;
        mt = fmaxf(mt, x[4 * kb + e]);
      }
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
    uint32_t pw[4];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = (x[e] == -INFINITY) ? 0.f : fast_exp2(x[e] - m_run);
      const float p1 = (x[e + 1] == -INFINITY) ? 0.f : fast_exp2(x[e + 1] - m_run);
      const uint32_t pk = pack_bf16x2(p0, p1);
      lsum += bf16lo(pk) + bf16hi(pk);
      pw[e >> 1] = pk;
    }
    l_run += lsum;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int blk = 0; blk < DBLK; ++blk) {
      if (rescale) oacc[blk] *= alpha;
      const int d = 16 * blk + vdofs;
      const int c = d >> 3, within = d & 7;
      const u32x2 lo = lds_read_tr16(vs + swz<D>(vkey0, c) + within);
      const u32x2 hi = lds_read_tr16(vs + swz<D>(16 + vkey0, c) + within);
      const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      oacc[blk] = mfma16x16x32(va, pb, oacc[blk]);
    }
    if (more) {
      stage_store(t + 1, buf ^ 1);
      mcur = mnxt;
    }
    __syncthreads();
  }

  float l_tot = l_run + lane_xor(l_run, 16);
  l_tot += lane_xor(l_tot, 32);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = (uint16_t*)p.out + ((b * p.Hq + h) * p.S_q + s) * (int64_t)D + 4 * grp;
#pragma unroll
    for (int blk = 0; blk < DBLK; ++blk) {
      u32x2 pk;
      pk.x = pack_bf16x2(oacc[blk][0] * inv, oacc[blk][1] * inv);
      pk.y = pack_bf16x2(oacc[blk][2] * inv, oacc[blk][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * blk) = pk;
    }
  }
}

template <int D, int NW, bool kRules, typename BiasT>
static hipError_t launch_prefill_inst(const AttnParams& p, hipStream_t stream) {
  constexpr bool k16 = D >= 512;   // 16-row wavefronts (see attn_prefill16_kernel)
  const int MQ = ((k16 ? 16 : 32) * NW) / p.G;
  const int n_qt = (p.S_q + MQ - 1) / MQ;
  const size_t lds = prefill_lds_bytes(D, p.T);
  void (*kern)(AttnParams, int);
  if constexpr (k16) kern = attn_prefill16_kernel<D, NW, kRules, BiasT>;
  else kern = attn_prefill_kernel<D, NW, kRules, BiasT>;
  // Opt in to the dynamic LDS this launch needs (static LDS of the kernel comes
  // on top, so the request is the exact size, not the CU's 160 KiB).
  {
    const hipError_t e = opt_in_dynamic_lds((const void*)kern, lds);
    if (e != hipSuccess) {
      set_launch_detail("hipFuncSetAttribute(MaxDynamicSharedMemorySize)");
      return e;
    }
  }
  const dim3 grid((unsigned)((int64_t)n_qt * p.B * p.Hkv));
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, stream, p, n_qt);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) set_launch_detail("prefill kernel launch");
  return e;
}

template <int D, int NW>
static hipError_t launch_prefill_v(const AttnParams& p, hipStream_t stream) {
  if (p.bias == nullptr) return launch_prefill_inst<D, NW, true, uint16_t>(p, stream);
  if (p.bias_is_bf16) return launch_prefill_inst<D, NW, false, uint16_t>(p, stream);
  return launch_prefill_inst<D, NW, false, uint32_t>(p, stream);
}

template <int D>
static hipError_t launch_prefill_d(const AttnParams& p, hipStream_t stream) {
  // 4 wavefronts (128 rows) when that still gives about one workgroup per CU,
  // else 2 (64 rows): more, smaller workgroups
  if constexpr (D >= 512) {
    return launch_prefill_v<D, 4>(p, stream);
  } else {
    const int64_t wg4 = (int64_t)p.B * p.Hkv * ((p.S_q * (int64_t)p.G + 127) / 128);
    if (wg4 >= 256) return launch_prefill_v<D, 4>(p, stream);
    return launch_prefill_v<D, 2>(p, stream);
  }
}

hipError_t launch_attn_prefill(const AttnParams& p, hipStream_t stream) {
  if (p.Dv != p.D)   // only the direct-to-LDS kernel has a V head size of its own
    return prefill_dma_supported(p) ? launch_attn_prefill_dma(p, stream) : hipErrorInvalidValue;
  // rows that allow 16-byte direct-to-LDS fetches take attn_prefill_dma.hip
  if (prefill_dma_supported(p)) return launch_attn_prefill_dma(p, stream);
  if (prefill_lds_bytes(p.D, p.T) > 160 * 1024) return hipErrorInvalidValue;
  switch (p.D) {
    case 64: return launch_prefill_d<64>(p, stream);
    case 128: return launch_prefill_d<128>(p, stream);
    case 256: return launch_prefill_d<256>(p, stream);
    case 512: return launch_prefill_d<512>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace abgqa
