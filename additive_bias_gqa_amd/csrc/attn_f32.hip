// fp32 attention over the static cache: one wavefront per query row.
//
// Pipeline (onnxruntime skill "cuda-attention-kernel-patterns", section 4):
// x_j = scale * (q . k_j) + bias_j, softmax over the kept keys, times V. A key
// is kept iff j < nonpad and bias_j != -inf (section 11 external cache; mobius
// issue #366); masked keys are removed by selection, and a row with no kept
// key writes zeros (section 6). Query head h reads KV head h / G (onnxruntime
// PR #28242, CPU GQA excerpt). Softmax is online, in base 2.
//
// This path serves fp32 inputs (small shapes, exactness at 1e-5); bf16 inputs
// use the matrix-core kernels.
#include "common.h"
#include "kernels.h"
#include "mask_rules.h"

namespace abgqa {

template <bool kRules, typename BiasT>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p, int64_t n_rows) {
  extern __shared__ float smem[];
  float* q_s = smem;            // [D]
  float* p_s = smem + p.D;      // [64]
  const int lane = threadIdx.x;
  const int D = p.D, T = p.T;
  const float* qg = (const float*)p.q;
  const float* kg = (const float*)p.k;
  const float* vg = (const float*)p.v;
  float* og = (float*)p.out;
  constexpr int kMaxDPerLane = 8;  // D <= 512
  const int d_per_lane = (D + 63) / 64;

  for (int64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
    const int s = (int)(row % p.S_q);
    const int h = (int)((row / p.S_q) % p.Hq);
    const int64_t b = row / ((int64_t)p.S_q * p.Hq);
    const int hk = h / p.G;
    const int64_t np = clamp_nonpad(p.nonpad[b], T);
    RowRule rule{};
    if constexpr (kRules) rule = make_row_rule(p.nonpad, p.q_start, p.slot_kind, b, s, p.S_q, T, p.window);
    const BiasT* brow = kRules ? nullptr : (const BiasT*)p.bias + (b * p.S_q + s) * T;
    const int32_t* krow = p.slot_kind ? p.slot_kind + b * T : nullptr;
    const float* kbase = kg + (b * p.Hkv + hk) * (int64_t)T * D;
    const float* vbase = vg + (b * p.Hkv + hk) * (int64_t)T * D;

    for (int d = lane; d < D; d += 64) q_s[d] = qg[row * D + d];
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
          const float* kr = kbase + j * D;
          float dot = 0.f;
          for (int d = 0; d < D; ++d) dot = fmaf(q_s[d], kr[d], dot);
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
          if (d < D) {
            for (int jj = 0; jj < nj; ++jj) {
              const float w = p_s[jj];
              if (w != 0.f) acc = fmaf(w, vbase[(j0 + jj) * D + d], acc);  // select, not multiply
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
      if (i < d_per_lane && d < D) og[row * D + d] = (l > 0.f) ? o[i] / l : 0.f;
    }
    __syncthreads();
  }
}

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) {
  const int64_t n_rows = (int64_t)p.B * p.Hq * p.S_q;
  int64_t blocks = n_rows < 65535 ? n_rows : 65535;
  const size_t lds = (size_t)(p.D + 64) * sizeof(float);
  if (p.bias == nullptr) {
    hipLaunchKernelGGL((attn_f32_kernel<true, float>), dim3((unsigned)blocks), dim3(64), lds, stream, p, n_rows);
  } else if (p.bias_is_bf16) {
    hipLaunchKernelGGL((attn_f32_kernel<false, uint16_t>), dim3((unsigned)blocks), dim3(64), lds, stream, p, n_rows);
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<false, float>), dim3((unsigned)blocks), dim3(64), lds, stream, p, n_rows);
  }
  return hipGetLastError();
}

}  // namespace abgqa
