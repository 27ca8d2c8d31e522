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
//   workgroup  one (b, kv head, query tile): 16*NW rows r = s_local * G + g,
//              i.e. MQ = 16*NW / G consecutive query tokens times the G heads
//              of the group. NW wavefronts own 16 rows each.
//   tiles      32 keys. The workgroup first lists its live tiles: tiles below
//              nonpad that hold an allowed entry for one of its rows (scanned
//              from the bias, or derived from the rules). Skipping a tile is
//              exact: every masked key contributes exactly zero.
//   LDS        per tile, K as [32][D+8] and V transposed as [D][32+4] (bf16),
//              double-buffered; each tile is read by all G heads' rows.
//   S^T = K Q^T    16x16x32 bf16 MFMA: A = K rows from LDS, B = Q^T held in
//                  registers for the whole loop. Result lane l: query row
//                  (l % 16), keys 4*(l/16) + e (+16 for the second half).
//   softmax        on that layout: a row's 32 scores sit in 4 lanes x 8 values;
//                  weights rounded to bf16 (RNE), the row sum adds the rounded
//                  weights. The running max moves only when exceeded by > 8.
//   O^T += V^T P^T 16x16x32 MFMA: A = V^T read from the transposed LDS tile,
//                  B = P^T straight from the softmax registers (its 8 k-slots
//                  are the 8 keys the lane holds). O^T lane l: query row l%16,
//                  d = 16*blk + 4*(l/16) + e.
#include "common.h"
#include "kernels.h"
#include "mask_rules.h"

namespace abgqa {

namespace {

constexpr int kTileKeys = 32;
constexpr float kRescaleThreshold = 8.f;

template <int D>
struct PrefillLds {
  static constexpr int KST = D + 8;                 // K row stride (bf16)
  static constexpr int VST = kTileKeys + 4;         // V^T row stride (bf16)
  static constexpr int K_ELEMS = kTileKeys * KST;
  static constexpr int V_ELEMS = D * VST;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr size_t BUF_BYTES = (size_t)BUF_ELEMS * 2;
};

__host__ __device__ inline int num_tiles(int n) { return (n + kTileKeys - 1) / kTileKeys; }

template <typename BiasT>
__device__ __forceinline__ bool live_bits(BiasT v);
template <>
__device__ __forceinline__ bool live_bits<uint16_t>(uint16_t v) { return v != 0xFF80; }
template <>
__device__ __forceinline__ bool live_bits<uint32_t>(uint32_t v) { return v != 0xFF800000u; }

}  // namespace

size_t prefill_lds_bytes(int D, int max_seq) {
  const int nt = num_tiles(max_seq);
  const size_t words = (size_t)((nt + 31) / 32) * 4;  // live bitmap
  const size_t list = (size_t)nt * 2;                 // live tile list (u16)
  const size_t buf = (size_t)(kTileKeys * (D + 8) + D * (kTileKeys + 4)) * 2;
  return 2 * buf + ((words + list + 15) & ~(size_t)15) + 64;
}

template <int D, int NW, bool kRules, typename BiasT>
__global__ __launch_bounds__(NW * 64) void attn_prefill_kernel(AttnParams p, int n_qt) {
  using L = PrefillLds<D>;
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 32;
  constexpr int DBLK = D / 16;
  constexpr int KCH = kTileKeys * (D / 8);   // 16-byte K chunks per tile
  constexpr int VUN = 8 * (D / 8);           // V units: 4 keys x 8 d
  constexpr int KPT = (KCH + NT - 1) / NT;   // K chunks per thread
  constexpr int VPT = (VUN + NT - 1) / NT;   // V units per thread

  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* bufs = reinterpret_cast<__bf16*>(smem);
  const int T = p.T, G = p.G;
  const int n_kt_max = num_tiles(T);
  uint32_t* s_bits = reinterpret_cast<uint32_t*>(smem + 2 * L::BUF_BYTES);
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
  const int qt = n_qt - 1 - (wg % n_qt);   // later (heavier) query tiles first
  const int bh = wg / n_qt;
  const int hk = bh % p.Hkv;
  const int64_t b = bh / p.Hkv;
  const int np = (int)clamp_nonpad(p.nonpad[b], T);
  const int MQ = (16 * NW) / G;
  const int s0 = qt * MQ;
  const int s_end = min(s0 + MQ, p.S_q);
  const int n_kt = num_tiles(np);

  // ---- 1. live tiles ---------------------------------------------------------
  for (int i = tid; i < n_words; i += NT) s_bits[i] = 0u;
  if (tid == 0) { s_nids = 0; s_nlive = 0; }
  if (tid < 4) s_ids[tid] = -1;  // never a block id: a racing reader cannot match it
  __syncthreads();
  if constexpr (!kRules) {
    constexpr int EPV = 16 / sizeof(BiasT);
    const int nvec = (np + EPV - 1) / EPV;
    const bool vec = (T % EPV) == 0;
    const BiasT* bb = (const BiasT*)p.bias + (b * p.S_q) * (int64_t)T;
    const int total = (s_end - s0) * nvec;
    for (int idx = tid; idx < total; idx += NT) {
      const int s = s0 + idx / nvec;
      const int j0 = (idx % nvec) * EPV;
      const BiasT* row = bb + (int64_t)s * T;
      BiasT vals[EPV];
      if (vec) {
        *reinterpret_cast<u32x4*>(vals) = ld_global<u32x4>(row + j0);
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) vals[e] = (j0 + e < T) ? row[j0 + e] : (BiasT)0;
      }
      bool any = false;
#pragma unroll
      for (int e = 0; e < EPV; ++e) any |= (j0 + e < np) && live_bits<BiasT>(vals[e]);
      if (any) {
        const int t = j0 / kTileKeys;   // EPV divides the tile size
        atomicOr(&s_bits[t >> 5], 1u << (t & 31));
      }
    }
  } else {
    // causal + window: keys [q_first - W + 1, q_last] (q consecutive over rows)
    if (tid == 0 && s_end > s0) {
      const RowRule r0 = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s0, p.S_q, T, p.window);
      const int64_t q_last = r0.q + (s_end - 1 - s0);
      int64_t a = (p.window > 0) ? r0.q - p.window + 1 : 0;
      if (a < 0) a = 0;
      const int64_t z = q_last < (int64_t)np - 1 ? q_last : (int64_t)np - 1;
      if (a <= z) {
        for (int t = (int)(a / kTileKeys); t <= (int)(z / kTileKeys); ++t)
          s_bits[t >> 5] |= 1u << (t & 31);
      }
    }
    // image blocks of the rows (up to 4 distinct ids; more: every tile is live)
    if (p.slot_kind) {
      for (int s = s0 + tid; s < s_end; s += NT) {
        const RowRule rr = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window);
        if (rr.kind_q > 0) {
          bool seen = false;
          for (int i = 0; i < 4; ++i) seen |= (i < s_nids) && (s_ids[i] == rr.kind_q);
          if (!seen) {
            const int slot = atomicAdd(&s_nids, 1);
            if (slot < 4) s_ids[slot] = rr.kind_q;
          }
        }
      }
    }
    __syncthreads();
    const int nids = s_nids;
    if (nids > 4) {
      for (int t = tid; t < n_kt; t += NT) atomicOr(&s_bits[t >> 5], 1u << (t & 31));
    } else if (nids > 0) {
      const int32_t* kr = p.slot_kind + b * T;
      for (int j = tid; j < np; j += NT) {
        const int32_t kj = kr[j];
        bool hit = false;
        for (int i = 0; i < nids; ++i) hit |= (kj == s_ids[i]);
        if (hit) atomicOr(&s_bits[(j / kTileKeys) >> 5], 1u << ((j / kTileKeys) & 31));
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
  const int n_live = s_nlive;

  // ---- 2. this lane's query row and its Q^T fragments ------------------------
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
    if (row_ok) rule = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window);
  }
  const BiasT* brow = kRules ? nullptr : (const BiasT*)p.bias + (b * p.S_q + (row_ok ? s : 0)) * (int64_t)T;
  const int32_t* kindb = p.slot_kind ? p.slot_kind + b * T : nullptr;
  const bool bias_vec = (T % 4) == 0;
  const float scale_log2 = p.scale * kLog2e;

  const __bf16* kg = (const __bf16*)p.k + (b * p.Hkv + hk) * (int64_t)T * D;
  const __bf16* vg = (const __bf16*)p.v + (b * p.Hkv + hk) * (int64_t)T * D;

  // ---- 3. tile staging: global -> registers -> LDS ---------------------------
  bf16x8 kreg[KPT];
  bf16x8 vreg[VPT][4];
  auto stage_load = [&](int t) {
    const int j0 = (int)s_list[t] * kTileKeys;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      const int kk = c / (D / 8), dc = c % (D / 8);
      const int j = j0 + kk;
      kreg[i] = (c < KCH && j < np) ? ld_global<bf16x8>(kg + (int64_t)j * D + 8 * dc) : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * NT;
      const int kgp = u % 8, dc = u / 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 4 * kgp + e;
        vreg[i][e] = (u < VUN && j < np) ? ld_global<bf16x8>(vg + (int64_t)j * D + 8 * dc) : bf16x8{};
      }
    }
  };
  auto stage_store = [&](int buf) {
    __bf16* ks = bufs + buf * L::BUF_ELEMS;
    __bf16* vt = ks + L::K_ELEMS;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (c < KCH) {
        const int kk = c / (D / 8), dc = c % (D / 8);
        *reinterpret_cast<bf16x8*>(ks + kk * L::KST + 8 * dc) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * NT;
      if (u < VUN) {
        const int kgp = u % 8, dc = u / 8;
        const u32x4 a0 = __builtin_bit_cast(u32x4, vreg[i][0]);
        const u32x4 a1 = __builtin_bit_cast(u32x4, vreg[i][1]);
        const u32x4 a2 = __builtin_bit_cast(u32x4, vreg[i][2]);
        const u32x4 a3 = __builtin_bit_cast(u32x4, vreg[i][3]);
        // d = 8*dc + e: the 4 keys' values of that d, packed key-consecutive
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int wi = e >> 1;
          const bool hi = e & 1;
          const uint32_t x0 = hi ? (a0[wi] >> 16) : (a0[wi] & 0xffffu);
          const uint32_t x1 = hi ? (a1[wi] >> 16) : (a1[wi] & 0xffffu);
          const uint32_t x2 = hi ? (a2[wi] >> 16) : (a2[wi] & 0xffffu);
          const uint32_t x3 = hi ? (a3[wi] >> 16) : (a3[wi] & 0xffffu);
          u32x2 pk;
          pk.x = x0 | (x1 << 16);
          pk.y = x2 | (x3 << 16);
          *reinterpret_cast<u32x2*>(vt + (8 * dc + e) * L::VST + 4 * kgp) = pk;
        }
      }
    }
  };

  // ---- 4. main loop ---------------------------------------------------------
  f32x4 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (n_live > 0) {
    stage_load(0);
    stage_store(0);
  }
  __syncthreads();
  for (int t = 0; t < n_live; ++t) {
    const int buf = t & 1;
    const int j0 = (int)s_list[t] * kTileKeys;
    if (t + 1 < n_live) stage_load(t + 1);

    // bias / rules for this lane's 8 keys: j0 + 16*kb + 4*grp + e
    float badd[2][4];
    bool keep[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int jb = j0 + 16 * kb + 4 * grp;
      if constexpr (kRules) {
        int32_t kv[4] = {0, 0, 0, 0};
        if (kindb) {
          if ((T % 4) == 0 && jb < T) {
            const int4 k4 = ld_global<int4>(kindb + jb);
            kv[0] = k4.x; kv[1] = k4.y; kv[2] = k4.z; kv[3] = k4.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) kv[e] = (jb + e < T) ? kindb[jb + e] : 0;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jb + e;
          keep[kb][e] = row_ok && (j < np) && rule.allowed(j, kv[e]);
          badd[kb][e] = 0.f;
        }
      } else {
        BiasT bv[4];
        if (row_ok && bias_vec && jb + 3 < T) {
          if constexpr (sizeof(BiasT) == 2) {
            const u32x2 raw = ld_global<u32x2>(brow + jb);
            bv[0] = raw.x & 0xffff; bv[1] = raw.x >> 16; bv[2] = raw.y & 0xffff; bv[3] = raw.y >> 16;
          } else {
            const u32x4 raw = ld_global<u32x4>(brow + jb);
            bv[0] = raw.x; bv[1] = raw.y; bv[2] = raw.z; bv[3] = raw.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) bv[e] = (row_ok && jb + e < T) ? brow[jb + e] : (BiasT)0;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jb + e;
          keep[kb][e] = row_ok && (j < np) && live_bits<BiasT>(bv[e]);
          float f;
          if constexpr (sizeof(BiasT) == 2) f = bf16_bits_to_f32(bv[e]);
          else f = __uint_as_float(bv[e]);
          badd[kb][e] = keep[kb][e] ? f * kLog2e : 0.f;
        }
      }
    }

    // S^T = K Q^T
    const __bf16* ks = bufs + buf * L::BUF_ELEMS;
    const __bf16* vt = ks + L::K_ELEMS;
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const __bf16* kr = ks + (16 * kb + col) * L::KST + 8 * grp;
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i)
        sacc[kb] = mfma16x16x32(*reinterpret_cast<const bf16x8*>(kr + 32 * i), qf[i], sacc[kb]);
    }

    // online softmax for query row `col` (values spread over the 4 groups)
    float x[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[kb][e] = keep[kb][e] ? fmaf(sacc[kb][e], scale_log2, badd[kb][e]) : -INFINITY;
        mt = fmaxf(mt, x[kb][e]);
      }
    mt = fmaxf(mt, lane_xor(mt, 16));
    mt = fmaxf(mt, lane_xor(mt, 32));
    const float mn = fmaxf(m_run, mt);
    const bool need = mn > m_run + kRescaleThreshold;
    if (__any(need)) {
      const float alpha = need ? fast_exp2(m_run - mn) : 1.f;
      if (need) m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) oacc[i] *= alpha;
    }
    uint32_t pw[4];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float p0 = (x[kb][e] == -INFINITY) ? 0.f : fast_exp2(x[kb][e] - m_run);
        const float p1 = (x[kb][e + 1] == -INFINITY) ? 0.f : fast_exp2(x[kb][e + 1] - m_run);
        const uint32_t pk = pack_bf16x2(p0, p1);
        lsum += bf16lo(pk) + bf16hi(pk);
        pw[2 * kb + (e >> 1)] = pk;
      }
    l_run += lsum;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});

    // O^T += V^T P^T
#pragma unroll
    for (int i = 0; i < DBLK; ++i) {
      const __bf16* vr = vt + (16 * i + col) * L::VST + 4 * grp;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
      const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      oacc[i] = mfma16x16x32(va, pb, oacc[i]);
    }

    if (t + 1 < n_live) stage_store(buf ^ 1);
    __syncthreads();
  }

  // ---- 5. normalise and store -----------------------------------------------
  float l_tot = l_run + lane_xor(l_run, 16);
  l_tot += lane_xor(l_tot, 32);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = (uint16_t*)p.out + ((b * p.Hq + h) * p.S_q + s) * (int64_t)D + 4 * grp;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) {
      u32x2 pk;
      pk.x = pack_bf16x2(oacc[i][0] * inv, oacc[i][1] * inv);
      pk.y = pack_bf16x2(oacc[i][2] * inv, oacc[i][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * i) = pk;
    }
  }
}

template <int D, int NW, bool kRules, typename BiasT>
static hipError_t launch_prefill_inst(const AttnParams& p, hipStream_t stream) {
  const int MQ = (16 * NW) / p.G;
  const int n_qt = (p.S_q + MQ - 1) / MQ;
  const size_t lds = prefill_lds_bytes(D, p.T);
  auto kern = attn_prefill_kernel<D, NW, kRules, BiasT>;
  // Opt in to the dynamic LDS this launch needs (static LDS of the kernel comes
  // on top, so the request is the exact size, not the CU's 160 KiB).
  static size_t lds_set = 0;  // per instantiation
  if (lds > lds_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
      set_launch_detail("hipFuncSetAttribute(MaxDynamicSharedMemorySize)");
      return e;
    }
    lds_set = lds;
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
  // 8 wavefronts (128 rows) when that still gives >= 2 workgroups per CU; at
  // D = 512 the 8-wavefront variant would spill (its O^T alone is 128 VGPRs)
  const int64_t wg8 = (int64_t)p.B * p.Hkv * ((p.S_q * (int64_t)p.G + 127) / 128);
  if (D < 512 && wg8 >= 512) return launch_prefill_v<D, 8>(p, stream);
  return launch_prefill_v<D, 4>(p, stream);
}

hipError_t launch_attn_prefill(const AttnParams& p, hipStream_t stream) {
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
