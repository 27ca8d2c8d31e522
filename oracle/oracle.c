/*
 * Plain fp64 CPU reference ("oracle") for additive-bias grouped-query attention
 * over an external static KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. The pytest suite, the smoke check and the CPU
 * baseline leg of the benchmark call it; the HIP library neither links nor calls
 * it, and it shares no code, header or table with that library.
 *
 * It is written to be checked by eye against the pages it follows, not to be
 * fast: every output element is computed straight from its definition, with no
 * tiling, no online softmax and no skipping. The only parallelism is an OpenMP
 * loop over independent output rows.
 *
 * Sources (the pages are cited by title and section):
 *   [I366] mobius issue #366, "Emit bias-aware external-KV (TensorScatter +
 *          nonpad_kv_seqlen) attention for float-bias decoders", sections
 *          "Problem" and "Mobius-side deliverable".
 *   [SKL]  onnxruntime skill "cuda-attention-kernel-patterns" (ONNX domain
 *          Attention opset 23/24), section 4 "Softcap Ordering", section 6
 *          "Fully-Masked Rows and Batches", section 8 "Cross-EP Consistency",
 *          section 11 "Causal Alignment".
 *   [OPT]  mobius skill "attention-optimization", sections "In-place KV for ONNX
 *          Attention via TensorScatter (static cache)" and "GQA sliding window
 *          via local_window_size".
 *   [PR]   onnxruntime PR #28242 "[GQA] ... add Gemma4 support", the CPU
 *          gqa_attention_base.h excerpt (query head i reads KV head
 *          i / kv_num_heads_factor).
 *
 * Parity pins: every function here is pinned by tests/test_oracle.py against
 * library routines, closed forms, hand-derived fixtures (tests/golden/) and
 * invariants; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* TensorScatter along the sequence axis of a [B, H, max_seq, D] cache.       */
/* [OPT] "In-place KV ... via TensorScatter": the new tokens are written into */
/* the fixed buffer at write_indices; nothing else changes. Element values    */
/* are copied as raw bytes (elem_bytes each), so the result is bit-exact for   */
/* any dtype. A destination slot outside [0, max_seq) is dropped (reading:    */
/* linear mode, no wrap-around). write_indices == NULL means all zero.        */
/* ------------------------------------------------------------------------- */
void oracle_scatter(unsigned char *cache, const unsigned char *update,
                    const int64_t *write_indices, int64_t B, int64_t H,
                    int64_t max_seq, int64_t S_new, int64_t D,
                    int64_t elem_bytes) {
  const int64_t row_bytes = D * elem_bytes;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t start = write_indices ? write_indices[b] : 0;
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t t = 0; t < S_new; ++t) {
        const int64_t slot = start + t;
        if (slot < 0 || slot >= max_seq) continue;
        unsigned char *dst = cache + ((b * H + h) * max_seq + slot) * row_bytes;
        const unsigned char *src = update + ((b * H + h) * S_new + t) * row_bytes;
        memcpy(dst, src, (size_t)row_bytes);
      }
    }
  }
}

/* ------------------------------------------------------------------------- */
/* Static-cache additive bias, shape [B, 1, S_q, max_seq], 0.0 or -inf.       */
/* [I366] "Mobius-side deliverable": a (B,1,S_q,max_seq) bias keyed on the    */
/* absolute query position, key validity slot < nonpad_kv_seqlen, combining   */
/* the causal, sliding-window, block-overlay and padding rules.               */
/*   query position  q = q_start[b] + s; default q_start = max(nonpad-S_q, 0)  */
/*                   ([SKL] section 11, bottom-right offset for an external   */
/*                   cache, clamped at zero);                                  */
/*   causal          key j <= q;                                               */
/*   window          keys [q-W+1, q] ([OPT] local_window_size, HF semantics);  */
/*                   W <= 0 means no window;                                   */
/*   block overlay   tokens of one image block (same positive slot kind) see   */
/*                   each other in both directions ([I366] "Problem",          */
/*                   Gemma-4 bidirectional vision-block overlay);              */
/*   padding         a pad slot (negative kind) is never a valid key;          */
/*   validity        j < nonpad[b] (nonpad clamped to [0, max_seq]).           */
/* allowed = valid && ((causal && window) || block). slot_kind == NULL means   */
/* every slot is text (kind 0). A query position outside [0, max_seq) has      */
/* kind 0. All position arithmetic is signed ([SKL] section 12).               */
/* ------------------------------------------------------------------------- */
void oracle_bias(double *bias, const int64_t *nonpad, const int64_t *q_start,
                 const int32_t *slot_kind, int64_t B, int64_t S_q,
                 int64_t max_seq, int64_t window) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t s = 0; s < S_q; ++s) {
      int64_t np = nonpad[b];
      if (np < 0) np = 0;
      if (np > max_seq) np = max_seq;
      int64_t qs;
      if (q_start) {
        qs = q_start[b];
      } else {
        qs = np - S_q;
        if (qs < 0) qs = 0;
      }
      const int64_t q = qs + s;
      int32_t kind_q = 0;
      if (slot_kind && q >= 0 && q < max_seq) kind_q = slot_kind[b * max_seq + q];
      double *row = bias + (b * S_q + s) * max_seq;
      for (int64_t j = 0; j < max_seq; ++j) {
        const int32_t kind_j = slot_kind ? slot_kind[b * max_seq + j] : 0;
        const int valid = (j < np) && (kind_j >= 0);
        const int causal = (j <= q);
        const int in_window = (window <= 0) || (q - j < window);
        const int block = (kind_q > 0) && (kind_j == kind_q);
        const int allowed = valid && ((causal && in_window) || block);
        row[j] = allowed ? 0.0 : -INFINITY;
      }
    }
  }
}

/* ------------------------------------------------------------------------- */
/* Materialise the KV heads for every query head: dst[b, h] = src[b, h / G].  */
/* [PR] CPU GQA excerpt: query head i reads KV head i / kv_num_heads_factor,  */
/* with G = Hq / Hkv contiguous query heads per KV head.                      */
/* ------------------------------------------------------------------------- */
void oracle_repeat_kv(double *dst, const double *src, int64_t B, int64_t Hkv,
                      int64_t G, int64_t T, int64_t D) {
  const int64_t Hq = Hkv * G;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < Hq; ++h)
      memcpy(dst + (b * Hq + h) * T * D, src + (b * Hkv + h / G) * T * D,
             (size_t)(T * D) * sizeof(double));
}

/* ------------------------------------------------------------------------- */
/* Dense multi-head attention with an additive bias broadcast over heads.     */
/* Q [B,H,S_q,D], K [B,H,T,D], V [B,H,T,Dv] (KV heads already repeated; the    */
/* value head size Dv may differ from D), bias [B,1,S_q,T], out [n_rows, Dv]  */
/* for the listed rows (row = (b*H + h)*S_q + s), or [B,H,S_q,Dv] when rows   */
/* == NULL.                                                                    */
/* [SKL] section 4: x_j = scale * (q . k_j), softcap when asked, then + bias, */
/* then softmax, then times V.                                                */
/* A key j is kept iff j < nonpad[b] and bias != -inf. Excluded keys are left  */
/* out by selection, so whatever K/V hold there never enters the arithmetic   */
/* ([SKL] section 6: select, not multiply).                                   */
/* A row with no kept key is written as zeros ([SKL] section 6, onnx#8068).   */
/* Softmax subtracts the row maximum first, as the CPU EP does ([SKL] §8).    */
/* ------------------------------------------------------------------------- */
void oracle_attention_mha(double *out, const double *q, const double *k,
                          const double *v, const double *bias,
                          const int64_t *nonpad, int64_t B, int64_t H,
                          int64_t S_q, int64_t T, int64_t D, int64_t Dv, double scale,
                          double softcap, const int64_t *rows, int64_t n_rows,
                          double *scratch /* [n_rows or B*H*S_q, T] */) {
  const int64_t total = rows ? n_rows : B * H * S_q;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < total; ++r) {
    const int64_t row = rows ? rows[r] : r;
    const int64_t s = row % S_q;
    const int64_t h = (row / S_q) % H;
    const int64_t b = row / (S_q * H);
    int64_t np = nonpad[b];
    if (np < 0) np = 0;
    if (np > T) np = T;
    const double *qr = q + ((b * H + h) * S_q + s) * D;
    const double *br = bias + (b * S_q + s) * T;
    double *x = scratch + r * T;
    double *o = out + r * Dv;

    /* scores of the kept keys; -inf marks an excluded key */
    double m = -INFINITY;
    int64_t kept = 0;
    for (int64_t j = 0; j < T; ++j) {
      const int keep = (j < np) && (br[j] != -INFINITY);
      if (!keep) {
        x[j] = -INFINITY;
        continue;
      }
      const double *kr = k + ((b * H + h) * T + j) * D;
      double dot = 0.0;
      for (int64_t d = 0; d < D; ++d) dot += qr[d] * kr[d];
      /* the skill page, section 4 "Softcap Ordering": stage 0 scale * QK^T,
         stage 1 softcap * tanh(. / softcap) when softcap > 0, stage 2 + bias */
      double sc = scale * dot;
      if (softcap > 0.0) sc = softcap * tanh(sc / softcap);
      x[j] = sc + br[j];
      if (x[j] > m) m = x[j];
      ++kept;
    }

    for (int64_t d = 0; d < Dv; ++d) o[d] = 0.0;
    if (kept == 0) continue; /* fully masked row: Y = 0 */

    double denom = 0.0;
    for (int64_t j = 0; j < T; ++j) {
      const int keep = (j < np) && (br[j] != -INFINITY);
      if (!keep) continue;
      const double w = exp(x[j] - m);
      denom += w;
      const double *vr = v + ((b * H + h) * T + j) * Dv;
      for (int64_t d = 0; d < Dv; ++d) o[d] += w * vr[d];
    }
    for (int64_t d = 0; d < Dv; ++d) o[d] /= denom;
  }
}

/* ------------------------------------------------------------------------- */
/* Circular (window-sized) cache. Reading of [OPT] "GQA sliding window via    */
/* local_window_size", which names a circular cache as a way to bound the     */
/* memory of a sliding-window layer but leaves its layout open:               */
/*   capacity C = max_seq slots; the token of absolute position p is written  */
/*   to slot p mod C; L = kv_len[b] counts the tokens written so far          */
/*   (absolute, may exceed C), so slot j holds the newest position p < L with */
/*   p = j (mod C), pos(j) = j + C * floor((L-1-j) / C), and is valid iff     */
/*   j < min(L, C).                                                           */
/* ------------------------------------------------------------------------- */

/* TensorScatter into a circular cache: update token t of batch row b has     */
/* absolute position write_pos[b] + t and lands in slot (that position) mod C; */
/* a negative position is dropped. Raw-byte copies. S_new <= C, so no two      */
/* tokens of one call share a slot.                                           */
void oracle_scatter_circular(unsigned char *cache, const unsigned char *update,
                             const int64_t *write_pos, int64_t B, int64_t H,
                             int64_t C, int64_t S_new, int64_t D,
                             int64_t elem_bytes) {
  const int64_t row_bytes = D * elem_bytes;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t start = write_pos ? write_pos[b] : 0;
    for (int64_t h = 0; h < H; ++h) {
      for (int64_t t = 0; t < S_new; ++t) {
        const int64_t p = start + t;
        if (p < 0) continue;
        const int64_t slot = p % C;
        unsigned char *dst = cache + ((b * H + h) * C + slot) * row_bytes;
        const unsigned char *src = update + ((b * H + h) * S_new + t) * row_bytes;
        memcpy(dst, src, (size_t)row_bytes);
      }
    }
  }
}

/* Bias [B, 1, S_q, C] of a circular cache: the rules of oracle_bias, applied  */
/* to the absolute position each slot holds.                                  */
/*   query position q = q_start[b] + s; default q_start = max(L - S_q, 0);    */
/*   its kind is that of slot q mod C when position q is still held           */
/*   (max(L - C, 0) <= q < L), else 0;                                        */
/*   key slot j: valid iff j < min(L, C) and kind_j >= 0; position pos(j);    */
/*   causal pos <= q; window q - pos < W (W <= 0: none); block kind_q > 0 and  */
/*   kind_j == kind_q; allowed = valid && ((causal && window) || block).      */
void oracle_bias_circular(double *bias, const int64_t *kv_len, const int64_t *q_start,
                          const int32_t *slot_kind, int64_t B, int64_t S_q,
                          int64_t C, int64_t window) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t s = 0; s < S_q; ++s) {
      int64_t L = kv_len[b];
      if (L < 0) L = 0;
      const int64_t n_valid = L < C ? L : C;
      const int64_t oldest = L > C ? L - C : 0;    /* oldest position still held */
      int64_t qs;
      if (q_start) {
        qs = q_start[b];
      } else {
        qs = L - S_q;
        if (qs < 0) qs = 0;
      }
      const int64_t q = qs + s;
      int32_t kind_q = 0;
      if (slot_kind && q >= oldest && q < L) kind_q = slot_kind[b * C + q % C];
      double *row = bias + (b * S_q + s) * C;
      for (int64_t j = 0; j < C; ++j) {
        if (j >= n_valid) {
          row[j] = -INFINITY;
          continue;
        }
        const int64_t pos = j + C * ((L - 1 - j) / C);
        const int32_t kind_j = slot_kind ? slot_kind[b * C + j] : 0;
        const int valid = kind_j >= 0;
        const int causal = pos <= q;
        const int in_window = (window <= 0) || (q - pos < window);
        const int block = (kind_q > 0) && (kind_j == kind_q);
        const int allowed = valid && ((causal && in_window) || block);
        row[j] = allowed ? 0.0 : -INFINITY;
      }
    }
  }
}
