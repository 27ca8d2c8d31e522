/*
 * abgqa.h - C ABI of libabgqa.so: additive-bias grouped-query attention over an
 * external static KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The computation is the opset-24 ONNX Attention op used as an external static
 * cache (onnxruntime skill "cuda-attention-kernel-patterns", section 11
 * "TensorScatter decode"; mobius skill "attention-optimization", section
 * "In-place KV for ONNX Attention via TensorScatter (static cache)"):
 *
 *   kv_tensor_scatter(K), kv_tensor_scatter(V)     write the new token(s)
 *   build_static_cache_bias(...)                   (B,1,S_q,max_seq) float bias
 *   attn_bias_gqa_fwd(Q, K, V, bias, nonpad, ...)  softmax(scale*QK^T + bias) V
 *
 * mobius issue #366, "Emit bias-aware external-KV (TensorScatter +
 * nonpad_kv_seqlen) attention for float-bias decoders", states the problem
 * these three calls solve. kv_scatter_and_bias does the first two in one
 * launch, attn_bias_gqa_decode_step all three for decode shapes; each has a
 * circular-cache form (*_circular), and attn_bias_gqa_fwd_noalloc is the
 * attention for callers that cannot allocate.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major (last index fastest), in caller-owned device
 *     memory, and 16-byte aligned. The library keeps no pointer after a call
 *     returns and allocates no device memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and runs asynchronously to the host. Return codes report host-side
 *     validation and launch errors only.
 *   - On any status other than ABGQA_OK nothing was enqueued, and
 *     abgqa_last_error() returns a stable one-line message (per thread).
 *   - Device-side index values (write_indices, nonpad_kv_seqlen, q_start) cannot
 *     be checked without a synchronisation; the kernels clamp nonpad into
 *     [0, max_seq] and drop writes outside the cache.
 *   - ABGQA_CHECK=1 in the environment (read at every call; skipped while the
 *     stream is being captured into a graph) makes every entry point
 *     synchronise its stream, copy those index arrays to the host and refuse,
 *     with ABGQA_ERR_INVALID and nothing enqueued, nonpad outside
 *     [0, max_seq], a negative q_start, or write_indices that put a new token
 *     outside [0, max_seq); a decode call also refuses a workspace whose
 *     arrival counts are not zero (ABGQA_ERR_WORKSPACE). After enqueuing, the
 *     call synchronises again and reports asynchronous errors (ABGQA_ERR_HIP).
 *   - Layout names: B batch, Hq query heads, Hkv KV heads (G = Hq / Hkv query
 *     heads share one KV head), S_q query tokens, max_seq cache slots, D head
 *     size. D must be one of 64, 128, 256, 512.
 */
#ifndef ABGQA_H
#define ABGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ABGQA_F32 = 0,  /* IEEE binary32 */
  ABGQA_BF16 = 1  /* bfloat16 (8-bit exponent, 7-bit mantissa) */
} abgqa_dtype;

typedef enum {
  ABGQA_OK = 0,
  ABGQA_ERR_INVALID = 1,     /* null pointer, bad size, misaligned pointer */
  ABGQA_ERR_UNSUPPORTED = 2, /* valid request the library does not implement */
  ABGQA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  ABGQA_ERR_HIP = 4          /* the HIP runtime reported an error */
} abgqa_status;

/*
 * kv_tensor_scatter - in-place TensorScatter of new tokens into a static cache.
 *
 * Passage: mobius skill "attention-optimization", section "In-place KV for ONNX
 * Attention via TensorScatter (static cache)": the new token(s) are written into
 * the pre-allocated buffer at write_indices, with no growing concatenation.
 * The scatter runs along the max_seq axis of this layout.
 *
 *   cache          [B, Hkv, max_seq, D] of `dtype`, updated in place
 *   update         [B, Hkv, S_new, D]   of `dtype`
 *   write_indices  [B] int64 on the device: update token t of batch row b goes
 *                  to slot write_indices[b] + t. NULL means all zero. A slot
 *                  outside [0, max_seq) is dropped (linear mode, no wrap).
 *   S_new == 0     is a no-op (a KV-shared layer has nothing to append,
 *                  onnxruntime PR #28242, kv_sequence_length = 0).
 * Every other slot keeps its bits. The copy is bit-exact.
 * Errors: ABGQA_ERR_INVALID for null cache/update (S_new > 0), non-positive
 * B/Hkv/max_seq/D, negative S_new, misalignment; ABGQA_ERR_UNSUPPORTED for
 * another dtype or a D that is not a multiple of 8.
 */
abgqa_status kv_tensor_scatter(void *cache, const void *update,
                               const int64_t *write_indices, int64_t B,
                               int64_t Hkv, int64_t max_seq, int64_t S_new,
                               int64_t D, abgqa_dtype dtype, void *stream);

/*
 * build_static_cache_bias - the (B,1,S_q,max_seq) additive bias of a static
 * cache, keyed on absolute query position.
 *
 * Passage: mobius issue #366, "Mobius-side deliverable" (second bullet): a bias
 * keyed on absolute query positions with KV validity slot < nonpad_kv_seqlen,
 * reusing the causal / sliding / block-overlay / padding logic. Window rule:
 * mobius skill "attention-optimization", "GQA sliding window via
 * local_window_size" (query q sees keys [q-W+1, q]). Default query offset:
 * onnxruntime skill "cuda-attention-kernel-patterns", section 11 (bottom-right
 * offset nonpad - S_q, clamped at 0).
 *
 *   bias             [B, 1, S_q, max_seq] of `bias_dtype`, fully written:
 *                    +0.0 where allowed, -inf where masked
 *   nonpad_kv_seqlen [B] int64 on the device (count of valid slots)
 *   q_start          [B] int64 on the device: query row s sits at absolute slot
 *                    q = q_start[b] + s. NULL means max(nonpad[b] - S_q, 0).
 *   slot_kind        [B, max_seq] int32 on the device: < 0 padding token, 0 text,
 *                    k > 0 a token of image block k. NULL means all text.
 *   window           W > 0: sliding window of W keys; W <= 0: none
 * allowed(b,s,j) = j < nonpad[b] && kind[j] >= 0
 *                  && ((j <= q && q - j < W) || (kind[q] > 0 && kind[j] == kind[q]))
 * (the window term is dropped when W <= 0; kind[q] is 0 when q is outside the
 * cache). Positions are signed 64-bit throughout.
 * Errors: ABGQA_ERR_INVALID for a null bias or nonpad, non-positive sizes,
 * misalignment; ABGQA_ERR_UNSUPPORTED for a bias dtype other than f32/bf16.
 */
abgqa_status build_static_cache_bias(void *bias, abgqa_dtype bias_dtype,
                                     const int64_t *nonpad_kv_seqlen,
                                     const int64_t *q_start,
                                     const int32_t *slot_kind, int64_t B,
                                     int64_t S_q, int64_t max_seq,
                                     int64_t window, void *stream);

/*
 * kv_scatter_and_bias - the whole per-step preparation in one launch:
 *   kv_tensor_scatter(k_cache, k_update, write_indices, ...),
 *   kv_tensor_scatter(v_cache, v_update, write_indices, ...),
 *   build_static_cache_bias(bias, bias_dtype, nonpad_kv_seqlen, q_start,
 *                           slot_kind, B, S_q, max_seq, window, ...).
 *
 * Passages: those of the three calls it stands for (mobius skill
 * "attention-optimization", "In-place KV for ONNX Attention via TensorScatter
 * (static cache)"; mobius issue #366, "Mobius-side deliverable"). The results
 * are bit-identical to the three separate calls; the bias reads no cache, so
 * the three pieces of work run side by side in one grid.
 *
 *   k_cache, v_cache    [B, Hkv, max_seq, D] of `dtype`, updated in place
 *   k_update, v_update  [B, Hkv, S_new, D] of `dtype`
 *   write_indices       [B] int64 on the device, or NULL (all zero)
 *   bias                [B, 1, S_q, max_seq] of `bias_dtype`, fully written; NULL
 *                       skips the bias (the in-kernel-rules variant needs none)
 *   nonpad_kv_seqlen, q_start, slot_kind, S_q, window: as build_static_cache_bias
 *                       (read only when bias != NULL)
 *   S_new == 0 skips both scatters (KV-shared layer).
 * Layout, alignment, ownership and device-side index handling are those of the
 * separate calls.
 * Errors: the union of the errors of the separate calls (ABGQA_ERR_INVALID for
 * null or misaligned pointers or bad sizes, ABGQA_ERR_UNSUPPORTED for dtypes or
 * row sizes they reject); nothing is enqueued on any error.
 */
abgqa_status kv_scatter_and_bias(void *k_cache, void *v_cache, const void *k_update,
                                 const void *v_update, const int64_t *write_indices,
                                 int64_t B, int64_t Hkv, int64_t max_seq, int64_t S_new,
                                 int64_t D, abgqa_dtype dtype, void *bias,
                                 abgqa_dtype bias_dtype, const int64_t *nonpad_kv_seqlen,
                                 const int64_t *q_start, const int32_t *slot_kind,
                                 int64_t S_q, int64_t window, void *stream);

/*
 * attn_bias_gqa_fwd - attention of S_q query tokens over the external cache.
 *
 * Passages: onnxruntime skill "cuda-attention-kernel-patterns", section 4
 * (scale*QK^T, then the optional softcap, then + bias, then softmax, then times V),
 * section 6 (a query row with no allowed key, or a batch row with nonpad = 0,
 * outputs zeros, decided by selection so masked V never leaks), section 11
 * (external cache: keys are the cache slots < nonpad_kv_seqlen); mobius issue
 * #366 (bias present with is_causal = 0: the bias carries the causal rule);
 * onnxruntime PR #28242, CPU GQA excerpt (query head h reads KV head h / G).
 *
 *   out              [B, Hq, S_q, D_v] of `dtype` (must not alias an input)
 *   q                [B, Hq, S_q, D] of `dtype`
 *   k_cache          [B, Hkv, max_seq, D] of `dtype`
 *   v_cache          [B, Hkv, max_seq, D_v] of `dtype`
 *   D, D_v           head sizes of Q/K and of V/out, each 64, 128, 256 or 512;
 *                    they may differ (head_size != v_head_size, the skill
 *                    page's dispatch table: KV-shared layers reading the V of a
 *                    layer with another head size). bf16 decode runs on the
 *                    matrix cores for D_v == D and for (D, D_v) = (256, 512) or
 *                    (512, 256), and so does bf16 prefill (for those two pairs
 *                    when Hq > Hkv, 8 <= max_seq <= 65536 and the bias rows,
 *                    or slot-kind rows, are whole 16-byte chunks); other
 *                    cases take a vector-ALU path (fp32 arithmetic) with the
 *                    same results.
 *   bias             [B, 1, S_q, max_seq] of `bias_dtype`, broadcast over heads;
 *                    -inf masks a key. NULL selects the in-kernel-rules variant:
 *                    the mask of build_static_cache_bias is evaluated inside the
 *                    attention kernel from nonpad, q_start, slot_kind and window,
 *                    with the same result as passing that bias.
 *   nonpad_kv_seqlen [B] int64 on the device
 *   q_start, slot_kind, window: read only when bias == NULL (see above)
 *   scale            multiplies q.k before the bias is added (1/sqrt(D) usually)
 *   softcap          > 0: the score becomes softcap * tanh(scale * q.k / softcap)
 *                    before the bias is added (skill page, section 4 "Softcap
 *                    Ordering": a -inf bias still removes its key); 0 = none
 *   dtype            ABGQA_BF16 (fp32 accumulation, softmax weights rounded to
 *                    bf16 for the matrix-core PV product in prefill) or
 *                    ABGQA_F32 (fp32 throughout)
 *   workspace        device scratch of at least attn_bias_gqa_workspace_bytes()
 *                    bytes for the same shape, 16-byte aligned. Its first
 *                    64 KiB are the decode kernel's arrival counts (one int32
 *                    per kv head and batch row): ZERO-FILL THEM ONCE when the
 *                    workspace is allocated; every call leaves them zero (a
 *                    prefill call never touches them, so one workspace can
 *                    serve both). Decode (S_q * Hq / Hkv <= 16) keeps one
 *                    partial softmax result per split workgroup after them,
 *                    and requires the workspace; the last of a row's splits
 *                    to finish merges that row's results (decode with more
 *                    than 16384 kv-head-and-batch-row pairs takes the vector
 *                    kernel instead and needs none).
 *                    Prefill with a bias tensor keeps a live-tile map after
 *                    the counts
 *                    (one bit per batch row, query tile and 32-key tile,
 *                    built by a pass over the bias before the attention
 *                    kernel); for prefill it is optional: with a smaller or
 *                    NULL workspace every workgroup scans its bias rows
 *                    itself (same result). Calls that share a workspace must
 *                    not overlap in time.
 * Slots >= nonpad may hold any bits (NaN/Inf included); they never reach the
 * arithmetic. K/V at slots < nonpad are expected to be finite: a key masked by
 * the bias gets the exact weight 0, and 0 times a finite V is 0.
 * Maskless static-cache Attention (no bias tensor; skill page section 11, the
 * onnx#8068 alignment; mobius issue #366, sibling #345): is_causal = 1 is
 * bias = NULL, q_start = NULL, slot_kind = NULL, window = 0 - query i sees key
 * j iff j <= i + max(nonpad - S_q, 0) and j < nonpad; is_causal = 0 passes in
 * addition q_start[b] = max_seq (every valid key precedes every query).
 * Errors: ABGQA_ERR_INVALID (null pointers, sizes, Hq % Hkv != 0, S_q > max_seq,
 * softcap negative or not finite, misalignment), ABGQA_ERR_UNSUPPORTED (D not in {64,128,256,512}, dtype pair
 * not supported), ABGQA_ERR_WORKSPACE, ABGQA_ERR_HIP.
 */
abgqa_status attn_bias_gqa_fwd(void *out, const void *q, const void *k_cache,
                               const void *v_cache, const void *bias,
                               abgqa_dtype bias_dtype,
                               const int64_t *nonpad_kv_seqlen,
                               const int64_t *q_start, const int32_t *slot_kind,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q,
                               int64_t max_seq, int64_t D, int64_t D_v,
                               float scale, float softcap, int64_t window,
                               abgqa_dtype dtype,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Circular (window-sized) cache - the same four calls for a cache whose
 * buffer is bounded by the window instead of the sequence.
 *
 * Passage: mobius skill "attention-optimization", section "GQA sliding window
 * via local_window_size": the window masks attention but does not shrink the
 * buffer, so bounding a sliding layer's memory takes a circular (or static)
 * cache. The page leaves the layout open; the layout taken here:
 *   capacity C (the max_seq of the layout names above) slots per (b, kv head);
 *   the token of absolute position p lives in slot p mod C;
 *   kv_len[b] = L, the count of tokens written so far (absolute, may exceed C,
 *   int64 on the device): slot j holds the newest position p < L with
 *   p = j (mod C) and is valid iff j < min(L, C);
 *   the static cache's rules (causal, window [q-W+1, q], image blocks, pads)
 *   apply to the absolute positions the slots hold and to the absolute query
 *   position q = q_start[b] + s (default q_start = max(L - S_q, 0)); a query's
 *   kind is that of slot q mod C while position q is held, else 0.
 * With C >= W + S_q - 1 every key a query of the chunk may see is still held,
 * and the results equal those of a static cache holding the same tokens.
 *
 * kv_tensor_scatter_circular: update token t of batch row b (position
 *   write_pos[b] + t) goes to slot (write_pos[b] + t) mod C; a negative
 *   position is dropped. S_new <= C (ABGQA_ERR_INVALID otherwise), so no two
 *   tokens of one call share a slot. Other arguments, errors and the bit-exact
 *   copy: those of kv_tensor_scatter.
 * build_circular_cache_bias: the [B, 1, S_q, C] bias (+0.0 / -inf) of the rule
 *   above, from kv_len; otherwise as build_static_cache_bias.
 * kv_scatter_and_bias_circular: both scatters and the bias in one launch, as
 *   kv_scatter_and_bias.
 * attn_bias_gqa_fwd_circular: the attention over a circular cache, with its
 *   bias tensor (then the same as attn_bias_gqa_fwd with nonpad = kv_len, which
 *   the kernels clamp to C) or, bias == NULL, with the rule above evaluated in
 *   the kernel; workspace as attn_bias_gqa_fwd (attn_bias_gqa_workspace_bytes
 *   with max_seq = C).
 * Under ABGQA_CHECK, kv_len must be >= 0 and write_pos >= 0 (no upper bound).
 */
abgqa_status kv_tensor_scatter_circular(void *cache, const void *update,
                                        const int64_t *write_pos, int64_t B,
                                        int64_t Hkv, int64_t capacity, int64_t S_new,
                                        int64_t D, abgqa_dtype dtype, void *stream);

abgqa_status build_circular_cache_bias(void *bias, abgqa_dtype bias_dtype,
                                       const int64_t *kv_len, const int64_t *q_start,
                                       const int32_t *slot_kind, int64_t B,
                                       int64_t S_q, int64_t capacity,
                                       int64_t window, void *stream);

abgqa_status kv_scatter_and_bias_circular(void *k_cache, void *v_cache,
                                          const void *k_update, const void *v_update,
                                          const int64_t *write_pos, int64_t B,
                                          int64_t Hkv, int64_t capacity, int64_t S_new,
                                          int64_t D, abgqa_dtype dtype, void *bias,
                                          abgqa_dtype bias_dtype, const int64_t *kv_len,
                                          const int64_t *q_start,
                                          const int32_t *slot_kind, int64_t S_q,
                                          int64_t window, void *stream);

abgqa_status attn_bias_gqa_fwd_circular(void *out, const void *q, const void *k_cache,
                                        const void *v_cache, const void *bias,
                                        abgqa_dtype bias_dtype, const int64_t *kv_len,
                                        const int64_t *q_start, const int32_t *slot_kind,
                                        int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q,
                                        int64_t capacity, int64_t D, int64_t D_v,
                                        float scale, float softcap, int64_t window,
                                        abgqa_dtype dtype, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * attn_bias_gqa_decode_step - one decode step in one launch: the TensorScatter
 * of the new K and V rows, the bias build and the attention.
 *
 * Passages: mobius skill "attention-optimization", "In-place KV for ONNX
 * Attention via TensorScatter (static cache)" (a step writes its new K/V rows
 * into the preallocated cache, then attends over it); mobius issue #366,
 * "Mobius-side deliverable" (the bias rules); the attention as
 * attn_bias_gqa_fwd.
 *
 * Results, bit for bit: those of
 *   kv_scatter_and_bias(k_cache, v_cache, k_update, v_update, write_indices,
 *                       B, Hkv, max_seq, S_new, ..., bias, bias_dtype,
 *                       nonpad_kv_seqlen, q_start, slot_kind, S_q, window)
 * followed by attn_bias_gqa_fwd with that bias (or, bias == NULL, with the
 * in-kernel rules, which give the same output): k_cache and v_cache hold the
 * new rows, bias (if not NULL) holds the [B, 1, S_q, max_seq] mask, out the
 * attention. The attention masks with the rules evaluated in the kernel, so it
 * does not wait for the bias; a key of a slot this call writes is taken from
 * the update rows.
 *   k_update, v_update [B, Hkv, S_new, D] and [B, Hkv, S_new, D_v] bf16
 *   (S_new = 0: no scatter, e.g. a KV-shared layer reading a borrowed
 *   cache); V rows may have their own head size, unlike kv_scatter_and_bias.
 *   Other arguments as kv_scatter_and_bias and attn_bias_gqa_fwd; workspace
 *   as attn_bias_gqa_fwd (required).
 * Shapes: bf16 decode shapes of the split-KV kernel only: S_q * Hq / Hkv <= 16,
 * D = D_v in {64, 128, 256, 512} or (D, D_v) = (256, 512) / (512, 256),
 * B * Hkv <= 16384, S_new <= 16; anything else is ABGQA_ERR_UNSUPPORTED (use
 * the separate calls). The call must not overlap other calls that read or
 * write the same caches or workspace.
 * Errors: those of kv_scatter_and_bias and attn_bias_gqa_fwd;
 * ABGQA_ERR_UNSUPPORTED as above.
 *
 * attn_bias_gqa_decode_step_circular: the same step over a circular cache of
 * capacity C (kv_tensor_scatter_circular, build_circular_cache_bias and
 * attn_bias_gqa_fwd_circular in one launch); S_new <= C.
 */
abgqa_status attn_bias_gqa_decode_step(void *out, const void *q, void *k_cache,
                                       void *v_cache, const void *k_update,
                                       const void *v_update,
                                       const int64_t *write_indices, int64_t S_new,
                                       void *bias, abgqa_dtype bias_dtype,
                                       const int64_t *nonpad_kv_seqlen,
                                       const int64_t *q_start, const int32_t *slot_kind,
                                       int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q,
                                       int64_t max_seq, int64_t D, int64_t D_v,
                                       float scale, float softcap, int64_t window,
                                       abgqa_dtype dtype, void *workspace,
                                       size_t workspace_bytes, void *stream);

abgqa_status attn_bias_gqa_decode_step_circular(void *out, const void *q, void *k_cache,
                                                void *v_cache, const void *k_update,
                                                const void *v_update,
                                                const int64_t *write_pos, int64_t S_new,
                                                void *bias, abgqa_dtype bias_dtype,
                                                const int64_t *kv_len,
                                                const int64_t *q_start,
                                                const int32_t *slot_kind, int64_t B,
                                                int64_t Hq, int64_t Hkv, int64_t S_q,
                                                int64_t capacity, int64_t D, int64_t D_v,
                                                float scale, float softcap, int64_t window,
                                                abgqa_dtype dtype, void *workspace,
                                                size_t workspace_bytes, void *stream);

/*
 * attn_bias_gqa_fwd_noalloc - attn_bias_gqa_fwd without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It allocates
 * nothing (no hipMalloc, hipFree or allocating library call).
 *
 *   Arguments, layouts, results and errors: those of attn_bias_gqa_fwd, with
 *   the same kernels and bit-identical outputs.
 *   Scratch: a library-owned static device array of 8 MiB (8388608 bytes) per
 *   GPU, held until the process ends; its address is looked up once per
 *   device. A shape whose attn_bias_gqa_workspace_bytes() exceeds 8 MiB is
 *   refused with ABGQA_ERR_WORKSPACE before anything is enqueued.
 *   The first call on a device clears the array's decode arrival counts with
 *   a small kernel on `stream` (a kernel node if the stream is being captured);
 *   every call leaves them zero again.
 *   Calls on one GPU share its array: calls that overlap in time on one GPU
 *   (concurrent streams or host threads) race and give wrong results.
 *   Calls ordered on one stream do not.
 */
abgqa_status attn_bias_gqa_fwd_noalloc(void *out, const void *q, const void *k_cache,
                                       const void *v_cache, const void *bias,
                                       abgqa_dtype bias_dtype,
                                       const int64_t *nonpad_kv_seqlen,
                                       const int64_t *q_start, const int32_t *slot_kind,
                                       int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q,
                                       int64_t max_seq, int64_t D, int64_t D_v,
                                       float scale, float softcap, int64_t window,
                                       abgqa_dtype dtype, void *stream);

/* Bytes of workspace attn_bias_gqa_fwd needs for this shape (0 if none). */
size_t attn_bias_gqa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv,
                                     int64_t S_q, int64_t max_seq, int64_t D,
                                     int64_t D_v);

/* Message of the last failed call on this thread ("" if none). The pointer stays
 * valid until the next call into the library from the same thread. */
const char *abgqa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ABGQA_H */
