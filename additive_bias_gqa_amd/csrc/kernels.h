// Internal launcher interface between the C ABI (abi.cpp) and the kernels.
// Arguments arrive validated: sizes positive, pointers non-null and aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace abgqa {

// Names the HIP call that failed inside a launcher (per thread; read and
// cleared by the C ABI when it reports ABGQA_ERR_HIP).
void set_launch_detail(const char* what);

// Opts kernel `kern` in to `lds` bytes of dynamic LDS on the current device
// (hipFuncSetAttribute, MaxDynamicSharedMemorySize), once per kernel, device
// and larger size; safe to call from several threads.
hipError_t opt_in_dynamic_lds(const void* kern, size_t lds);

// circular: a circular cache of capacity max_seq (mask_rules.h): the scatter
// writes position p to slot p mod max_seq, the bias takes nonpad as the
// absolute count of tokens written
hipError_t launch_scatter(void* cache, const void* update, const int64_t* write_indices,
                          int64_t B, int64_t H, int64_t max_seq, int64_t S_new,
                          int64_t row_bytes, bool circular, hipStream_t stream);

hipError_t launch_bias(void* bias, int bias_is_bf16, const int64_t* nonpad,
                       const int64_t* q_start, const int32_t* slot_kind, int64_t B,
                       int64_t S_q, int64_t max_seq, int64_t window, bool circular,
                       hipStream_t stream);

// grid sizes of the two (capped, grid-stride)
int64_t scatter_blocks(int64_t n_rows, int vec_per_row);
int64_t bias_blocks(int64_t B, int64_t S_q, int64_t max_seq);

// K scatter + V scatter + bias build in one launch (prepare.hip); S_new == 0
// skips the scatters, bias == null skips the bias.
hipError_t launch_prepare(void* k_cache, void* v_cache, const void* k_update, const void* v_update,
                          const int64_t* write_indices, int64_t B, int64_t H, int64_t max_seq,
                          int64_t S_new, int64_t row_bytes, void* bias, int bias_is_bf16,
                          const int64_t* nonpad, const int64_t* q_start, const int32_t* slot_kind,
                          int64_t S_q, int64_t window, bool circular, hipStream_t stream);

// Everything an attention kernel reads, passed by value.
// The first bytes of every attention workspace: the decode kernel's arrival
// counts, one int per (kv head, batch row). They must be zero before the first
// call that uses the workspace; every call leaves them zero. The rest of the
// workspace (decode partial records, prefill live-tile map) follows.
constexpr size_t kWsCounterBytes = 64 * 1024;
constexpr int64_t kMaxDecodeRows = (int64_t)(kWsCounterBytes / sizeof(int));

struct AttnParams {
  void* out;                 // [B, Hq, S_q, Dv]
  const void* q;             // [B, Hq, S_q, D]
  const void* k;             // [B, Hkv, T, D]
  const void* v;             // [B, Hkv, T, Dv]
  const void* bias;          // [B, 1, S_q, T] or null (in-kernel rules)
  const int64_t* nonpad;     // [B]
  const int64_t* q_start;    // [B] or null (rules variant only)
  const int32_t* slot_kind;  // [B, T] or null (rules variant only)
  int B, Hq, Hkv, G, S_q, T, D;
  int Dv;                    // head size of V and the output
  int64_t window;            // rules variant only; <= 0 none
  float scale;               // multiplies q.k
  float softcap;             // > 0: softcap * tanh(scale * q.k / softcap) before the bias
  int bias_is_bf16;          // bias dtype when bias != null
  int circular;              // circular cache: nonpad is the absolute count of
                             // tokens written, position p in slot p mod T
  // split-KV decode
  float* ws_part;            // partial results, one record per (b, kv head, split)
  int* arrive;               // split arrivals per (kv head, b): zero between calls
  int n_split;
  // prefill: caller scratch (may be null); the direct-to-LDS path keeps its
  // live-tile map there when it is large enough
  void* ws;
  size_t ws_bytes;
  // prefill, bias variant: live-tile map [B][query tiles][words] built by a
  // pass over the bias before the attention kernel, or null (each workgroup
  // then scans its bias rows itself)
  const uint32_t* tilemap;
  // one fused decode step (attn_decode_step.hip): before the attention reads
  // them, the S_new update rows [B, Hkv, S_new, D] / [.., DV] go into k / v at
  // write_idx[b] + t (TensorScatter; circular: that position mod T), and the
  // [B, 1, S_q, T] bias of the rules is written to bias_out (null: not written)
  const void* k_upd;
  const void* v_upd;
  const int64_t* write_idx;  // [B] or null (all 0)
  int S_new;
  void* bias_out;
  int bias_out_bf16;
};

// fp32 path (any S_q): one wavefront per query row.
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);
// the same computation for bf16 inputs (fp32 arithmetic, bf16 output): the
// path for head sizes the matrix-core kernels are not built for
hipError_t launch_attn_vec_bf16(const AttnParams& p, hipStream_t stream);

// bf16 decode path (S_q * G <= 16): one split-KV kernel; the last split of each
// row merges the row's partial results.
int decode_num_splits(int64_t B, int64_t Hkv, int64_t max_seq);
size_t decode_workspace_bytes(int64_t B, int64_t Hkv, int64_t S_q, int64_t G, int64_t Dv,
                              int64_t max_seq);
bool decode_supports(int D, int Dv);
hipError_t launch_attn_decode(const AttnParams& p, hipStream_t stream);
// the fused decode step: TensorScatter of K and V, the bias build and the
// attention (rules variant) in one launch of the split-KV kernel; the same
// shapes as launch_attn_decode, S_new <= 16
hipError_t launch_decode_step(const AttnParams& p, hipStream_t stream);

// bf16 prefill path: matrix-core tiles, K/V tiles in LDS shared by the G heads.
// Returns hipErrorInvalidValue when the shape needs more LDS than a CU has.
hipError_t launch_attn_prefill(const AttnParams& p, hipStream_t stream);
// direct-to-LDS prefill pipeline (attn_prefill_dma.hip) and when it applies
// (the only prefill path for D != Dv: D = 256 with Dv = 512, or the reverse)
bool prefill_dma_supported(const AttnParams& p);
// longest cache the direct-to-LDS prefill takes (its live-tile list lives in LDS)
constexpr int kDmaMaxSeq = 65536;
hipError_t launch_attn_prefill_dma(const AttnParams& p, hipStream_t stream);
// scratch bytes the prefill path can use for this shape (its live-tile map)
size_t prefill_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q, int64_t max_seq,
                               int64_t D, int64_t D_v);
// the same kernel with 32-row wavefronts and Q^T in registers
// (attn_prefill_dma_wide.hip): D = 512 with nw = 4, D = 256 with nw = 2 or 4,
// and the (D, Dv) pairs (256, 512) and (512, 256) with nw = 4 (their 16-row
// form is in attn_prefill_dma.hip)
hipError_t launch_attn_prefill_dma_qreg(const AttnParams& p, int nw, hipStream_t stream);
size_t prefill_lds_bytes(int D, int max_seq);

}  // namespace abgqa
