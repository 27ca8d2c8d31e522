// TensorScatter into the static KV cache (bit-exact 16-byte copies).
//
// mobius skill "attention-optimization", section "In-place KV for ONNX
// Attention via TensorScatter (static cache)": the new token(s) land in the
// pre-allocated buffer at write_indices[b] + t; nothing else is touched.
// Grid-stride over rows with a capped grid (onnxruntime skill
// "cuda-attention-kernel-patterns", section 5). Body: prep_device.h.
#include "common.h"
#include "kernels.h"
#include "prep_device.h"

namespace abgqa {

__global__ __launch_bounds__(256) void scatter_kernel(
    u32x4* __restrict__ cache, const u32x4* __restrict__ update,
    const int64_t* __restrict__ write_indices, int H, int max_seq, int S_new,
    int vec_per_row, int64_t n_rows, bool circular) {
  scatter_rows(cache, update, nullptr, nullptr, write_indices, H, max_seq, S_new, vec_per_row,
               n_rows, blockIdx.x, gridDim.x, circular);
}

int64_t scatter_blocks(int64_t n_rows, int vec_per_row) {
  const int rows_per_iter = 256 / vec_per_row;
  int64_t blocks = (n_rows + rows_per_iter - 1) / rows_per_iter;
  const int64_t kMaxBlocks = 65535;
  return blocks > kMaxBlocks ? kMaxBlocks : blocks;
}

hipError_t launch_scatter(void* cache, const void* update, const int64_t* write_indices,
                          int64_t B, int64_t H, int64_t max_seq, int64_t S_new,
                          int64_t row_bytes, bool circular, hipStream_t stream) {
  const int vec_per_row = (int)(row_bytes / 16);
  const int64_t n_rows = B * H * S_new;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)scatter_blocks(n_rows, vec_per_row)), dim3(256), 0,
                     stream, (u32x4*)cache, (const u32x4*)update, write_indices, (int)H,
                     (int)max_seq, (int)S_new, vec_per_row, n_rows, circular);
  return hipGetLastError();
}

}  // namespace abgqa
