// The per-step preparation in one launch: TensorScatter of the new K rows,
// TensorScatter of the new V rows (same write_indices), and the static-cache
// bias build. The three results are exactly those of kv_tensor_scatter (K),
// kv_tensor_scatter (V) and build_static_cache_bias; the bias does not read
// the caches, so the three pieces of work are independent and share a grid:
// workgroups [0, n_scatter) copy rows (each thread 16 bytes of K and the same
// 16 bytes of V), the rest build bias chunks. A decode step otherwise spends
// more time launching these three small kernels than running them.
#include "common.h"
#include "kernels.h"
#include "prep_device.h"

namespace abgqa {

template <typename T>
__global__ __launch_bounds__(256) void prepare_kernel(
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, const u32x4* __restrict__ k_update,
    const u32x4* __restrict__ v_update, const int64_t* __restrict__ write_indices, int H,
    int max_seq, int S_new, int vec_per_row, int64_t n_rows, int n_scatter, T* __restrict__ bias,
    const int64_t* __restrict__ nonpad, const int64_t* __restrict__ q_start,
    const int32_t* __restrict__ slot_kind, int S_q, int64_t window, int chunks_per_row,
    int64_t n_chunks, bool vec, bool circular) {
  if ((int)blockIdx.x < n_scatter) {
    scatter_rows(k_cache, k_update, v_cache, v_update, write_indices, H, max_seq, S_new,
                 vec_per_row, n_rows, blockIdx.x, n_scatter, circular);
  } else {
    bias_chunks<T>(bias, nonpad, q_start, slot_kind, S_q, max_seq, window, chunks_per_row, n_chunks,
                   vec, blockIdx.x - n_scatter, gridDim.x - n_scatter, circular);
  }
}

hipError_t launch_prepare(void* k_cache, void* v_cache, const void* k_update, const void* v_update,
                          const int64_t* write_indices, int64_t B, int64_t H, int64_t max_seq,
                          int64_t S_new, int64_t row_bytes, void* bias, int bias_is_bf16,
                          const int64_t* nonpad, const int64_t* q_start, const int32_t* slot_kind,
                          int64_t S_q, int64_t window, bool circular, hipStream_t stream) {
  const int vec_per_row = (int)(row_bytes / 16);
  const int64_t n_rows = B * H * S_new;
  const int n_scatter = S_new > 0 ? (int)scatter_blocks(n_rows, vec_per_row) : 0;
  const int n_bias = bias ? (int)bias_blocks(B, S_q, max_seq) : 0;
  if (n_scatter + n_bias == 0) return hipSuccess;
  const int chunks_per_row = (int)((max_seq + 7) / 8);
  const int64_t n_chunks = bias ? B * S_q * chunks_per_row : 0;
  const bool vec = (max_seq % 8) == 0;
  const dim3 grid((unsigned)(n_scatter + n_bias));
  if (!bias || bias_is_bf16) {
    hipLaunchKernelGGL(prepare_kernel<uint16_t>, grid, dim3(256), 0, stream, (u32x4*)k_cache,
                       (u32x4*)v_cache, (const u32x4*)k_update, (const u32x4*)v_update,
                       write_indices, (int)H, (int)max_seq, (int)S_new, vec_per_row, n_rows,
                       n_scatter, (uint16_t*)bias, nonpad, q_start, slot_kind, (int)S_q, window,
                       chunks_per_row, n_chunks, vec, circular);
  } else {
    hipLaunchKernelGGL(prepare_kernel<uint32_t>, grid, dim3(256), 0, stream, (u32x4*)k_cache,
                       (u32x4*)v_cache, (const u32x4*)k_update, (const u32x4*)v_update,
                       write_indices, (int)H, (int)max_seq, (int)S_new, vec_per_row, n_rows,
                       n_scatter, (uint32_t*)bias, nonpad, q_start, slot_kind, (int)S_q, window,
                       chunks_per_row, n_chunks, vec, circular);
  }
  return hipGetLastError();
}

}  // namespace abgqa
