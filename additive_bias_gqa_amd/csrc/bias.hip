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
// Body: prep_device.h.
#include "common.h"
#include "kernels.h"
#include "prep_device.h"

namespace abgqa {

template <typename T>
__global__ __launch_bounds__(256) void bias_kernel(
    T* __restrict__ bias, const int64_t* __restrict__ nonpad,
    const int64_t* __restrict__ q_start, const int32_t* __restrict__ slot_kind,
    int S_q, int max_seq, int64_t window, int chunks_per_row, int64_t n_chunks, bool vec,
    bool circular) {
  bias_chunks<T>(bias, nonpad, q_start, slot_kind, S_q, max_seq, window, chunks_per_row, n_chunks,
                 vec, blockIdx.x, gridDim.x, circular);
}

int64_t bias_blocks(int64_t B, int64_t S_q, int64_t max_seq) {
  const int64_t n_chunks = B * S_q * ((max_seq + 7) / 8);
  int64_t blocks = (n_chunks + 255) / 256;
  const int64_t kMaxBlocks = 65535;
  return blocks > kMaxBlocks ? kMaxBlocks : blocks;
}

hipError_t launch_bias(void* bias, int bias_is_bf16, const int64_t* nonpad,
                       const int64_t* q_start, const int32_t* slot_kind, int64_t B,
                       int64_t S_q, int64_t max_seq, int64_t window, bool circular,
                       hipStream_t stream) {
  const int chunks_per_row = (int)((max_seq + 7) / 8);
  const int64_t n_chunks = B * S_q * chunks_per_row;
  const bool vec = (max_seq % 8) == 0;
  const dim3 grid((unsigned)bias_blocks(B, S_q, max_seq));
  if (bias_is_bf16) {
    hipLaunchKernelGGL(bias_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       (uint16_t*)bias, nonpad, q_start, slot_kind, (int)S_q, (int)max_seq,
                       window, chunks_per_row, n_chunks, vec, circular);
  } else {
    hipLaunchKernelGGL(bias_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       (uint32_t*)bias, nonpad, q_start, slot_kind, (int)S_q, (int)max_seq,
                       window, chunks_per_row, n_chunks, vec, circular);
  }
  return hipGetLastError();
}

}  // namespace abgqa
