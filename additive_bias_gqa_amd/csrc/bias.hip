// Static-cache additive bias builder: (B, 1, S_q, max_seq), +0.0 or -inf.
//
// mobius issue #366, "Mobius-side deliverable": the bias is keyed on the
// absolute query position and marks a key valid iff slot < nonpad_kv_seqlen,
// combining the causal, sliding-window, block-overlay and padding rules.
// Sliding window: mobius skill "attention-optimization", "GQA sliding window
// via local_window_size" (keys [q-W+1, q]). Default query offset: onnxruntime
// skill "cuda-attention-kernel-patterns", section 11 (nonpad - S_q, clamped at
// 0). Positions are signed 64-bit (same skill, section 12).
//
// The same predicate is evaluated inside the attention kernels when no bias
// tensor is passed (mask_rules.h), so both variants agree bit for bit.
#include "common.h"
#include "kernels.h"
#include "mask_rules.h"

namespace abgqa {

// bits of +0.0 / -inf in the output type
template <typename T> struct MaskBits;
template <> struct MaskBits<uint16_t> {
  static constexpr uint16_t kZero = 0x0000, kNegInf = 0xFF80;
};
template <> struct MaskBits<uint32_t> {
  static constexpr uint32_t kZero = 0x00000000u, kNegInf = 0xFF800000u;
};

// One thread writes 8 consecutive keys of one (b, s) row. `vec` is true when
// every row starts 16-byte aligned (max_seq % 8 == 0), so kinds are read and
// bias written with 16-byte accesses.
template <typename T>
__global__ __launch_bounds__(256) void bias_kernel(
    T* __restrict__ bias, const int64_t* __restrict__ nonpad,
    const int64_t* __restrict__ q_start, const int32_t* __restrict__ slot_kind,
    int S_q, int max_seq, int64_t window, int chunks_per_row, int64_t n_chunks, bool vec) {
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n_chunks;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / chunks_per_row;
    const int j0 = (int)(idx - row * chunks_per_row) * 8;
    const int64_t b = row / S_q;
    const int s = (int)(row - b * S_q);
    const RowRule rule = make_row_rule(nonpad, q_start, slot_kind, b, s, S_q, max_seq, window);
    const int32_t* kind_row = slot_kind ? slot_kind + b * max_seq : nullptr;
    T* out = bias + row * max_seq + j0;
    if (vec) {
      int32_t kinds[8];
      if (kind_row) {
        const int4 k0 = ld_global<int4>(kind_row + j0);
        const int4 k1 = ld_global<int4>(kind_row + j0 + 4);
        kinds[0] = k0.x; kinds[1] = k0.y; kinds[2] = k0.z; kinds[3] = k0.w;
        kinds[4] = k1.x; kinds[5] = k1.y; kinds[6] = k1.z; kinds[7] = k1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kinds[e] = 0;
      }
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

hipError_t launch_bias(void* bias, int bias_is_bf16, const int64_t* nonpad,
                       const int64_t* q_start, const int32_t* slot_kind, int64_t B,
                       int64_t S_q, int64_t max_seq, int64_t window, hipStream_t stream) {
  const int chunks_per_row = (int)((max_seq + 7) / 8);
  const int64_t n_chunks = B * S_q * chunks_per_row;
  const bool vec = (max_seq % 8) == 0;
  int64_t blocks = (n_chunks + 255) / 256;
  const int64_t kMaxBlocks = 65535;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (bias_is_bf16) {
    hipLaunchKernelGGL(bias_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (uint16_t*)bias, nonpad, q_start, slot_kind, (int)S_q, (int)max_seq,
                       window, chunks_per_row, n_chunks, vec);
  } else {
    hipLaunchKernelGGL(bias_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (uint32_t*)bias, nonpad, q_start, slot_kind, (int)S_q, (int)max_seq,
                       window, chunks_per_row, n_chunks, vec);
  }
  return hipGetLastError();
}

}  // namespace abgqa
