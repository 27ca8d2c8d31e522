// fp32 attention over the static cache: one wavefront per query row.
//
// Pipeline (onnxruntime skill "cuda-attention-kernel-patterns", section 4):
// x_j = scale * (q . k_j) + bias_j, softmax over the kept keys, times V. A key
// is kept iff j < nonpad and bias_j != -inf (section 11 external cache; mobius
// issue #366); masked keys are removed by selection, and a row with no kept
// key writes zeros (section 6). Query head h reads KV head h / G (onnxruntime
// PR #28242, CPU GQA excerpt). Softmax is online, in base 2.
//
// This path serves fp32 inputs (small shapes, exactness at 1e-5). Built for
// bf16 inputs as well (fp32 arithmetic, the output rounded to bf16 once), it
// is the path for head-size pairs the matrix-core kernels are not built for;
// Q and K have head size D, V and the output Dv (which may differ: onnxruntime
// skill "cuda-attention-kernel-patterns", the head_size != v_head_size rows of
// its dispatch table).
#include "common.h"
#include "kernels.h"
#include "mask_rules.h"

namespace abgqa {

// element loads and stores: fp32, or bf16 held as its 16 bits
__device__ __forceinline__ float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_elem(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ void st_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_elem(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }

template <typename Elem, bool kRules, typename BiasT>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p, int64_t n_rows) {
  extern __shared__ float smem[];
  float* q_s = smem;            // [D]
  float* p_s = smem + p.D;      // [64]
  const int lane = threadIdx.x;
  const int D = p.D, Dv = p.Dv, T = p.T;
  const Elem* qg = (const Elem*)p.q;
  const Elem* kg = (const Elem*)p.k;
  const Elem* vg = (const Elem*)p.v;
  Elem* og = (Elem*)p.out;
  constexpr int kMaxDPerLane = 8;  // Dv <= 512
  const int d_per_lane = (Dv + 63) / 64;

  for (int64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
    const int s = (int)(row % p.S_q);
    const int h = (int)((row / p.S_q) % p.Hq);
    const int64_t b = row / ((int64_t)p.S_q * p.Hq);
    const int hk = h / p.G;
    const int64_t np = clamp_nonpad(p.nonpad[b], T);
    RowRule rule{};
    if constexpr (kRules) rule = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window, p.circular);
    const BiasT* brow = kRules ? nullptr : (const BiasT*)p.bias + (b * p.S_q + s) * T;
    const int32_t* krow = p.slot_kind ? p.slot_kind + b * T : nullptr;
    const Elem* kbase = kg + (b * p.Hkv + hk) * (int64_t)T * D;
    const Elem* vbase = vg + (b * p.Hkv + hk) * (int64_t)T * Dv;

    for (int d = lane; d < D; d += 64) q_s[d] = ld_elem(qg, row * D + d);
    __syncthreads();

    float o[kMaxDPerLane];
#pragma unroll
    for (int i = 0; i < kMaxDPerLane; ++i) o[i] = 0.f;
    float m = -INFINITY, l = 0.f;

    for (int64_t j0 = 0; j0 < np; j0 += 64) {
      const int64_t j = j0 + lane;
      float x = -INFINITY;
      if (j < np) {
        bool keep;
        float bv = 0.f;
        if constexpr (kRules) {
          keep = rule.allowed(j, krow ? krow[j] : 0);
        } else {
          if constexpr (sizeof(BiasT) == 2) bv = bf16_bits_to_f32(brow[j]);
          else bv = brow[j];
          keep = bv != -INFINITY;
        }
        if (keep) {
          const Elem* kr = kbase + j * D;
          float dot = 0.f;
          for (int d = 0; d < D; ++d) dot = fmaf(q_s[d], ld_elem(kr, d), dot);
          float sc = dot * p.scale;
          // softcap (skill page, section 4): before the bias; 0 = none
          if (p.softcap > 0.f) sc = p.softcap * tanhf(sc / p.softcap);
          x = (sc + bv) * kLog2e;
        }
      }
      const float m_new = fmaxf(m, wave_max(x));
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
      const float pj = (x == -INFINITY) ? 0.f : fast_exp2(x - m_new);
      l = l * alpha + wave_sum(pj);
      m = m_new;
      p_s[lane] = pj;
      __syncthreads();
      const int nj = (int)((np - j0) < 64 ? (np - j0) : 64);
#pragma unroll
      for (int i = 0; i < kMaxDPerLane; ++i) {
        if (i < d_per_lane) {
          const int d = lane + 64 * i;
          float acc = o[i] * alpha;
          if (d < Dv) {
            for (int jj = 0; jj < nj; ++jj) {
              const float w = p_s[jj];
              if (w != 0.f) acc = fmaf(w, ld_elem(vbase, (j0 + jj) * Dv + d), acc);  // select, not multiply
            }
          }
          o[i] = acc;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kMaxDPerLane; ++i) {
      const int d = lane + 64 * i;
      if (i < d_per_lane && d < Dv) st_elem(og, row * Dv + d, (l > 0.f) ? o[i] / l : 0.f);
    }
    __syncthreads();
  }
}

template <typename Elem>
static hipError_t launch_vec(const AttnParams& p, hipStream_t stream) {
  const int64_t n_rows = (int64_t)p.B * p.Hq * p.S_q;
  int64_t blocks = n_rows < 65535 ? n_rows : 65535;
  const size_t lds = (size_t)(p.D + 64) * sizeof(float);
  if (p.bias == nullptr) {
    hipLaunchKernelGGL((attn_f32_kernel<Elem, true, float>), dim3((unsigned)blocks), dim3(64), lds, stream, p,
                       n_rows);
  } else if (p.bias_is_bf16) {
    hipLaunchKernelGGL((attn_f32_kernel<Elem, false, uint16_t>), dim3((unsigned)blocks), dim3(64), lds, stream,
                       p, n_rows);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<Elem, false, float>), dim3((unsigned)blocks), dim3(64), lds, stream, p,
                       n_rows);
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) { return launch_vec<float>(p, stream); }
hipError_t launch_attn_vec_bf16(const AttnParams& p, hipStream_t stream) {
  return launch_vec<uint16_t>(p, stream);
}

}  // namespace abgqa
