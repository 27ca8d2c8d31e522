// TensorScatter into the static KV cache (bit-exact 16-byte copies).
//
// mobius skill "attention-optimization", section "In-place KV for ONNX
// Attention via TensorScatter (static cache)": the new token(s) land in the
// pre-allocated buffer at write_indices[b] + t; nothing else is touched.
// Grid-stride over rows with a capped grid (onnxruntime skill
// "cuda-attention-kernel-patterns", section 5).
#include "common.h"
#include "kernels.h"

namespace abgqa {

// One thread moves 16 bytes. A workgroup covers `rows_per_iter` update rows per
// iteration, each row being `vec_per_row` 16-byte vectors (1 <= vec_per_row <=
// 256); threads beyond rows_per_iter * vec_per_row idle.
__global__ __launch_bounds__(256) void scatter_kernel(
    u32x4* __restrict__ cache, const u32x4* __restrict__ update,
    const int64_t* __restrict__ write_indices, int H, int max_seq, int S_new,
    int vec_per_row, int64_t n_rows) {
  const int rows_per_iter = 256 / vec_per_row;
  const int sub = threadIdx.x / vec_per_row;
  const int c = threadIdx.x % vec_per_row;
  if (sub >= rows_per_iter) return;
  for (int64_t row = (int64_t)blockIdx.x * rows_per_iter + sub; row < n_rows;
       row += (int64_t)gridDim.x * rows_per_iter) {
    const int64_t bh = row / S_new;
    const int t = (int)(row - bh * S_new);
    const int64_t b = bh / H;
    const int64_t slot = (write_indices ? write_indices[b] : 0) + t;
    if (slot < 0 || slot >= max_seq) continue;  // dropped (no wrap-around)
    cache[(bh * max_seq + slot) * vec_per_row + c] = update[row * vec_per_row + c];
  }
}

hipError_t launch_scatter(void* cache, const void* update, const int64_t* write_indices,
                          int64_t B, int64_t H, int64_t max_seq, int64_t S_new,
                          int64_t row_bytes, hipStream_t stream) {
  const int vec_per_row = (int)(row_bytes / 16);
  const int64_t n_rows = B * H * S_new;
  const int rows_per_iter = 256 / vec_per_row;
  int64_t blocks = (n_rows + rows_per_iter - 1) / rows_per_iter;
  const int64_t kMaxBlocks = 65535;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (u32x4*)cache, (const u32x4*)update, write_indices, (int)H,
                     (int)max_seq, (int)S_new, vec_per_row, n_rows);
  return hipGetLastError();
}

}  // namespace abgqa
