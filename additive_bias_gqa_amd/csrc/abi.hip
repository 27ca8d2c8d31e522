// C ABI of libabgqa.so: host-side validation and dispatch. See include/abgqa.h
// for the contract of each entry point and the passages it follows.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "abgqa.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;
thread_local std::string g_launch_detail;

abgqa_status fail(abgqa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

abgqa_status hip_fail(const char* what, hipError_t e) {
  const std::string detail = g_launch_detail.empty() ? std::string() : " in " + g_launch_detail;
  g_launch_detail.clear();
  return fail(ABGQA_ERR_HIP, "%s: HIP error %d (%s)%s", what, (int)e, hipGetErrorString(e),
              detail.c_str());
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool log_enabled() {
  static const bool on = [] {
    const char* v = getenv("ABGQA_LOG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

constexpr int64_t kMaxSeq = (int64_t)1 << 24;  // slot indices stay exact in int32

// ABGQA_CHECK=1: before enqueuing, synchronise the stream, copy the device-side
// index arrays to the host and validate them; after enqueuing, synchronise
// again and report any asynchronous HIP error. Read at every call. Skipped while
// the stream is being captured into a graph (no synchronisation is allowed then).
bool check_requested() {
  const char* v = getenv("ABGQA_CHECK");
  return v && v[0] && v[0] != '0';
}

bool check_enabled(hipStream_t st) {
  if (!check_requested()) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs == hipStreamCaptureStatusNone;
}

// The n values of a device array, after the work already on `st` has finished.
// Fails (returns a status) if the pointer is not device-accessible memory or a
// HIP call fails.
abgqa_status fetch_device(const void* dptr, size_t bytes, void* host, hipStream_t st, const char* me,
                          const char* what) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, dptr) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ABGQA_ERR_INVALID, "%s: ABGQA_CHECK: %s is not device-accessible memory", me, what);
  }
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(me, e);
  e = hipMemcpy(host, dptr, bytes, hipMemcpyDefault);
  if (e != hipSuccess) return hip_fail(me, e);
  return ABGQA_OK;
}

abgqa_status fetch_i64(const int64_t* dptr, int64_t n, std::vector<int64_t>& out, hipStream_t st,
                       const char* me, const char* what) {
  out.assign((size_t)n, 0);
  return fetch_device(dptr, (size_t)n * sizeof(int64_t), out.data(), st, me, what);
}

// nonpad_kv_seqlen[b] in [0, max_seq] for every batch row (a circular cache:
// kv_len[b] >= 0, the count of tokens written may exceed the capacity)
abgqa_status check_nonpad(const int64_t* nonpad, int64_t B, int64_t max_seq, hipStream_t st,
                          const char* me, bool circular = false) {
  std::vector<int64_t> v;
  abgqa_status r = fetch_i64(nonpad, B, v, st, me, circular ? "kv_len" : "nonpad_kv_seqlen");
  if (r != ABGQA_OK) return r;
  for (int64_t b = 0; b < B; ++b)
    if (circular && v[b] < 0)
      return fail(ABGQA_ERR_INVALID, "%s: ABGQA_CHECK: kv_len[%lld] = %lld is negative", me,
                  (long long)b, (long long)v[b]);
    else if (!circular && (v[b] < 0 || v[b] > max_seq))
      return fail(ABGQA_ERR_INVALID,
                  "%s: ABGQA_CHECK: nonpad_kv_seqlen[%lld] = %lld is outside [0, max_seq = %lld]", me,
                  (long long)b, (long long)v[b], (long long)max_seq);
  return ABGQA_OK;
}

// q_start[b] >= 0: a query sits at a cache position
abgqa_status check_q_start(const int64_t* q_start, int64_t B, hipStream_t st, const char* me) {
  if (!q_start) return ABGQA_OK;
  std::vector<int64_t> v;
  abgqa_status r = fetch_i64(q_start, B, v, st, me, "q_start");
  if (r != ABGQA_OK) return r;
  for (int64_t b = 0; b < B; ++b)
    if (v[b] < 0)
      return fail(ABGQA_ERR_INVALID, "%s: ABGQA_CHECK: q_start[%lld] = %lld is negative", me,
                  (long long)b, (long long)v[b]);
  return ABGQA_OK;
}

// every written slot write_indices[b] + t, t < S_new, inside [0, max_seq)
// (a circular cache: every position >= 0)
abgqa_status check_write_indices(const int64_t* wi, int64_t B, int64_t max_seq, int64_t S_new,
                                 hipStream_t st, const char* me, bool circular = false) {
  if (!wi || S_new == 0) return S_new <= max_seq ? ABGQA_OK
                                                 : fail(ABGQA_ERR_INVALID,
                                                        "%s: ABGQA_CHECK: S_new = %lld slots past max_seq = %lld",
                                                        me, (long long)S_new, (long long)max_seq);
  std::vector<int64_t> v;
  abgqa_status r = fetch_i64(wi, B, v, st, me, "write_indices");
  if (r != ABGQA_OK) return r;
  for (int64_t b = 0; b < B; ++b)
    if (v[b] < 0 || (!circular && v[b] > max_seq - S_new))
      return fail(ABGQA_ERR_INVALID,
                  "%s: ABGQA_CHECK: write_indices[%lld] = %lld puts slots of the %lld new tokens "
                  "outside [0, max_seq = %lld)",
                  me, (long long)b, (long long)v[b], (long long)S_new, (long long)max_seq);
  return ABGQA_OK;
}

// after the launch: wait for it and report what went wrong asynchronously
abgqa_status check_after(hipStream_t st, const char* me) {
  const hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(me, e);
  return ABGQA_OK;
}

bool head_dim_ok(int64_t D) { return D == 64 || D == 128 || D == 256 || D == 512; }

}  // namespace

void abgqa::set_launch_detail(const char* what) { g_launch_detail = what; }

hipError_t abgqa::opt_in_dynamic_lds(const void* kern, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> done;   // (kernel, device) -> bytes
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = done[{kern, dev}];
  if (lds <= have) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) have = lds;
  return e;
}

namespace {

abgqa_status scatter_impl(const char* me, bool circular, void* cache, const void* update,
                          const int64_t* write_indices, int64_t B, int64_t Hkv, int64_t max_seq,
                          int64_t S_new, int64_t D, abgqa_dtype dtype, void* stream) {
  g_last_error.clear();
  if (B <= 0 || Hkv <= 0 || max_seq <= 0 || D <= 0)
    return fail(ABGQA_ERR_INVALID, "%s: B, Hkv, max_seq and D must be positive", me);
  if (S_new < 0) return fail(ABGQA_ERR_INVALID, "%s: S_new must be >= 0", me);
  if (circular && S_new > max_seq)
    return fail(ABGQA_ERR_INVALID, "%s: a circular cache takes at most capacity = %lld new tokens per call",
                me, (long long)max_seq);
  if (max_seq > kMaxSeq) return fail(ABGQA_ERR_UNSUPPORTED, "%s: max_seq above 2^24", me);
  if (dtype != ABGQA_F32 && dtype != ABGQA_BF16)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: dtype must be ABGQA_F32 or ABGQA_BF16", me);
  const int64_t row_bytes = D * (dtype == ABGQA_F32 ? 4 : 2);
  if (row_bytes % 16 != 0 || row_bytes > 4096)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: D * element size must be a multiple of 16 bytes, at most 4096", me);
  if (S_new == 0) return ABGQA_OK;  // nothing to append
  if (!cache || !update) return fail(ABGQA_ERR_INVALID, "%s: null cache or update", me);
  if (!aligned(cache, 16) || !aligned(update, 16) || (write_indices && !aligned(write_indices, 8)))
    return fail(ABGQA_ERR_INVALID, "%s: misaligned pointer", me);
  const hipStream_t st = (hipStream_t)stream;
  const bool chk = check_enabled(st);
  if (chk) {
    const abgqa_status r = check_write_indices(write_indices, B, max_seq, S_new, st, me, circular);
    if (r != ABGQA_OK) return r;
  }
  const hipError_t e = abgqa::launch_scatter(cache, update, write_indices, B, Hkv, max_seq, S_new,
                                             row_bytes, circular, st);
  if (e != hipSuccess) return hip_fail(me, e);
  return chk ? check_after(st, me) : ABGQA_OK;
}

abgqa_status bias_impl(const char* me, bool circular, void* bias, abgqa_dtype bias_dtype,
                       const int64_t* nonpad_kv_seqlen, const int64_t* q_start,
                       const int32_t* slot_kind, int64_t B, int64_t S_q, int64_t max_seq,
                       int64_t window, void* stream) {
  g_last_error.clear();
  if (B <= 0 || S_q <= 0 || max_seq <= 0)
    return fail(ABGQA_ERR_INVALID, "%s: B, S_q and max_seq must be positive", me);
  if (max_seq > kMaxSeq) return fail(ABGQA_ERR_UNSUPPORTED, "%s: max_seq above 2^24", me);
  if (bias_dtype != ABGQA_F32 && bias_dtype != ABGQA_BF16)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: bias dtype must be ABGQA_F32 or ABGQA_BF16", me);
  if (!bias || !nonpad_kv_seqlen)
    return fail(ABGQA_ERR_INVALID, "%s: null bias or nonpad_kv_seqlen", me);
  if (!aligned(bias, 16) || !aligned(nonpad_kv_seqlen, 8) || (q_start && !aligned(q_start, 8)) ||
      (slot_kind && !aligned(slot_kind, 16)))
    return fail(ABGQA_ERR_INVALID, "%s: misaligned pointer", me);
  const hipStream_t st = (hipStream_t)stream;
  const bool chk = check_enabled(st);
  if (chk) {
    abgqa_status r = check_nonpad(nonpad_kv_seqlen, B, max_seq, st, me, circular);
    if (r == ABGQA_OK) r = check_q_start(q_start, B, st, me);
    if (r != ABGQA_OK) return r;
  }
  const hipError_t e = abgqa::launch_bias(bias, bias_dtype == ABGQA_BF16, nonpad_kv_seqlen, q_start,
                                          slot_kind, B, S_q, max_seq, window, circular, st);
  if (e != hipSuccess) return hip_fail(me, e);
  return chk ? check_after(st, me) : ABGQA_OK;
}

abgqa_status prepare_impl(const char* me, bool circular, void* k_cache, void* v_cache,
                          const void* k_update, const void* v_update, const int64_t* write_indices,
                          int64_t B, int64_t Hkv, int64_t max_seq, int64_t S_new, int64_t D,
                          abgqa_dtype dtype, void* bias, abgqa_dtype bias_dtype,
                          const int64_t* nonpad_kv_seqlen, const int64_t* q_start,
                          const int32_t* slot_kind, int64_t S_q, int64_t window, void* stream) {
  g_last_error.clear();
  if (B <= 0 || Hkv <= 0 || max_seq <= 0 || D <= 0)
    return fail(ABGQA_ERR_INVALID, "%s: B, Hkv, max_seq and D must be positive", me);
  if (S_new < 0) return fail(ABGQA_ERR_INVALID, "%s: S_new must be >= 0", me);
  if (circular && S_new > max_seq)
    return fail(ABGQA_ERR_INVALID, "%s: a circular cache takes at most capacity = %lld new tokens per call",
                me, (long long)max_seq);
  if (max_seq > kMaxSeq) return fail(ABGQA_ERR_UNSUPPORTED, "%s: max_seq above 2^24", me);
  if (dtype != ABGQA_F32 && dtype != ABGQA_BF16)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: dtype must be ABGQA_F32 or ABGQA_BF16", me);
  const int64_t row_bytes = D * (dtype == ABGQA_F32 ? 4 : 2);
  if (row_bytes % 16 != 0 || row_bytes > 4096)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: D * element size must be a multiple of 16 bytes, at most 4096", me);
  if (S_new > 0) {
    if (!k_cache || !v_cache || !k_update || !v_update)
      return fail(ABGQA_ERR_INVALID, "%s: null cache or update", me);
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_update, 16) ||
        !aligned(v_update, 16) || (write_indices && !aligned(write_indices, 8)))
      return fail(ABGQA_ERR_INVALID, "%s: misaligned cache, update or write_indices", me);
  }
  if (bias) {
    if (S_q <= 0) return fail(ABGQA_ERR_INVALID, "%s: S_q must be positive", me);
    if (bias_dtype != ABGQA_F32 && bias_dtype != ABGQA_BF16)
      return fail(ABGQA_ERR_UNSUPPORTED, "%s: bias dtype must be ABGQA_F32 or ABGQA_BF16", me);
    if (!nonpad_kv_seqlen) return fail(ABGQA_ERR_INVALID, "%s: null nonpad_kv_seqlen", me);
    if (!aligned(bias, 16) || !aligned(nonpad_kv_seqlen, 8) || (q_start && !aligned(q_start, 8)) ||
        (slot_kind && !aligned(slot_kind, 16)))
      return fail(ABGQA_ERR_INVALID, "%s: misaligned bias, nonpad, q_start or slot_kind", me);
  }
  if (S_new == 0 && !bias) return ABGQA_OK;  // nothing to do
  const hipStream_t st = (hipStream_t)stream;
  const bool chk = check_enabled(st);
  if (chk) {
    abgqa_status r = S_new > 0 ? check_write_indices(write_indices, B, max_seq, S_new, st, me, circular)
                               : ABGQA_OK;
    if (r == ABGQA_OK && bias) r = check_nonpad(nonpad_kv_seqlen, B, max_seq, st, me, circular);
    if (r == ABGQA_OK && bias) r = check_q_start(q_start, B, st, me);
    if (r != ABGQA_OK) return r;
  }
  const hipError_t e = abgqa::launch_prepare(k_cache, v_cache, k_update, v_update, write_indices, B,
                                             Hkv, max_seq, S_new, row_bytes, bias,
                                             bias_dtype == ABGQA_BF16, nonpad_kv_seqlen, q_start,
                                             slot_kind, S_q, window, circular, st);
  if (e != hipSuccess) return hip_fail(me, e);
  return chk ? check_after(st, me) : ABGQA_OK;
}

}  // namespace

extern "C" {

size_t attn_bias_gqa_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q,
                                     int64_t max_seq, int64_t D, int64_t D_v) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_q <= 0 || max_seq <= 0 || D <= 0 || D_v <= 0 || Hq % Hkv)
    return 0;
  const int64_t G = Hq / Hkv;
  if (S_q * G > 16) {
    const size_t map = abgqa::prefill_workspace_bytes(B, Hq, Hkv, S_q, max_seq, D, D_v);
    return map ? abgqa::kWsCounterBytes + map : 0;
  }
  if (!abgqa::decode_supports((int)D, (int)D_v) || B * Hkv > abgqa::kMaxDecodeRows) return 0;
  return abgqa::decode_workspace_bytes(B, Hkv, S_q, G, D_v, max_seq);
}

}  // extern "C"

namespace {

// The split-KV decode kernel's workspace: its size for the shape in p, its
// alignment, and under ABGQA_CHECK its arrival counts (zero between calls);
// then p's split count and workspace pointers.
abgqa_status decode_workspace(const char* me, abgqa::AttnParams& p, void* workspace,
                              size_t workspace_bytes, hipStream_t st, bool chk) {
  const size_t need = abgqa::decode_workspace_bytes(p.B, p.Hkv, p.S_q, p.G, p.Dv, p.T);
  if (!workspace || workspace_bytes < need)
    return fail(ABGQA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", me,
                need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(ABGQA_ERR_INVALID, "%s: workspace not 16-byte aligned", me);
  if (chk) {
    // the arrival counts this call uses must be zero
    std::vector<int32_t> cnt((size_t)p.B * p.Hkv);
    const abgqa_status r = fetch_device(workspace, cnt.size() * sizeof(int32_t), cnt.data(), st, me,
                                        "workspace");
    if (r != ABGQA_OK) return r;
    for (size_t i = 0; i < cnt.size(); ++i)
      if (cnt[i] != 0)
        return fail(ABGQA_ERR_WORKSPACE,
                    "%s: ABGQA_CHECK: decode arrival count %zu of the workspace is %d, "
                    "not 0 (workspace not zero-filled, or a call on it did not complete)",
                    me, i, (int)cnt[i]);
  }
  p.n_split = abgqa::decode_num_splits(p.B, p.Hkv, p.T);
  p.arrive = (int*)workspace;
  p.ws_part = (float*)((char*)workspace + abgqa::kWsCounterBytes);
  return ABGQA_OK;
}

abgqa_status attn_impl(const char* me, bool circular, void* out, const void* q, const void* k_cache,
                       const void* v_cache, const void* bias, abgqa_dtype bias_dtype,
                       const int64_t* nonpad_kv_seqlen, const int64_t* q_start,
                       const int32_t* slot_kind, int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q,
                       int64_t max_seq, int64_t D, int64_t D_v, float scale, float softcap,
                       int64_t window, abgqa_dtype dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_q <= 0 || max_seq <= 0 || D <= 0 || D_v <= 0)
    return fail(ABGQA_ERR_INVALID, "%s: B, Hq, Hkv, S_q, max_seq, D and D_v must be positive", me);
  if (Hq % Hkv != 0) return fail(ABGQA_ERR_INVALID, "%s: Hq must be a multiple of Hkv", me);
  if (!(softcap >= 0.f) || softcap == INFINITY)
    return fail(ABGQA_ERR_INVALID, "%s: softcap must be finite and >= 0 (0 = none)", me);
  if (S_q > max_seq) return fail(ABGQA_ERR_INVALID, "%s: S_q must not exceed max_seq", me);
  if (!head_dim_ok(D) || !head_dim_ok(D_v))
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: D and D_v must be 64, 128, 256 or 512", me);
  if (max_seq > kMaxSeq) return fail(ABGQA_ERR_UNSUPPORTED, "%s: max_seq above 2^24", me);
  if (dtype != ABGQA_F32 && dtype != ABGQA_BF16)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: dtype must be ABGQA_F32 or ABGQA_BF16", me);
  if (bias && bias_dtype != ABGQA_F32 && bias_dtype != ABGQA_BF16)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: bias dtype must be ABGQA_F32 or ABGQA_BF16", me);
  if (!out || !q || !k_cache || !v_cache || !nonpad_kv_seqlen)
    return fail(ABGQA_ERR_INVALID, "%s: null out, q, k_cache, v_cache or nonpad_kv_seqlen", me);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      (bias && !aligned(bias, 16)) || !aligned(nonpad_kv_seqlen, 8) || (q_start && !aligned(q_start, 8)) ||
      (slot_kind && !aligned(slot_kind, 16)))
    return fail(ABGQA_ERR_INVALID, "%s: misaligned pointer", me);
  if (out == q || out == k_cache || out == v_cache || out == bias)
    return fail(ABGQA_ERR_INVALID, "%s: out must not alias an input", me);
  const int64_t G = Hq / Hkv;
  if (B * Hq * S_q > ((int64_t)1 << 31) || B * Hkv > ((int64_t)1 << 24))
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: too many rows", me);

  abgqa::AttnParams p{};
  p.out = out; p.q = q; p.k = k_cache; p.v = v_cache; p.bias = bias;
  p.nonpad = nonpad_kv_seqlen; p.q_start = q_start; p.slot_kind = slot_kind;
  p.B = (int)B; p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.G = (int)G; p.S_q = (int)S_q;
  p.T = (int)max_seq; p.D = (int)D; p.Dv = (int)D_v; p.window = window; p.scale = scale; p.softcap = softcap;
  p.bias_is_bf16 = (bias_dtype == ABGQA_BF16);
  p.circular = circular ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  const bool chk = check_enabled(st);
  if (chk) {
    abgqa_status r = check_nonpad(nonpad_kv_seqlen, B, max_seq, st, me, circular);
    if (r == ABGQA_OK && !bias) r = check_q_start(q_start, B, st, me);
    if (r != ABGQA_OK) return r;
  }

  hipError_t e;
  const char* path;
  if (dtype == ABGQA_F32) {
    path = "f32";
    e = abgqa::launch_attn_f32(p, st);
  } else if ((S_q * G <= 16 && (!abgqa::decode_supports((int)D, (int)D_v) || B * Hkv > abgqa::kMaxDecodeRows)) ||
             (S_q * G > 16 && D != D_v && !abgqa::prefill_dma_supported(p))) {
    // head sizes the matrix-core kernels are not built for, or more (b, kv
    // head) pairs than the decode arrival counts cover: the vector path
    path = "vector";
    e = abgqa::launch_attn_vec_bf16(p, st);
  } else if (S_q * G <= 16) {
    path = "decode";
    const abgqa_status r = decode_workspace(me, p, workspace, workspace_bytes, st, chk);
    if (r != ABGQA_OK) return r;
    e = abgqa::launch_attn_decode(p, st);
  } else {
    path = "prefill";
    if (G > 64) return fail(ABGQA_ERR_UNSUPPORTED, "%s: more than 64 query heads per KV head", me);
    // live key tiles are numbered in 16 bits and listed in LDS beside the K/V stages
    if ((max_seq + 31) / 32 > 65535 ||
        abgqa::prefill_lds_bytes((int)(D > D_v ? D : D_v), (int)max_seq) > 160 * 1024)
      return fail(ABGQA_ERR_UNSUPPORTED, "%s: max_seq too large for the prefill tile list", me);
    if (workspace && !aligned(workspace, 16))
      return fail(ABGQA_ERR_INVALID, "%s: workspace not 16-byte aligned", me);
    // optional here: with less than attn_bias_gqa_workspace_bytes() the
    // kernel finds its live tiles from the bias itself. The decode arrival
    // counts at the start of the workspace are left alone.
    const bool have = workspace && workspace_bytes > abgqa::kWsCounterBytes;
    p.ws = have ? (void*)((char*)workspace + abgqa::kWsCounterBytes) : nullptr;
    p.ws_bytes = have ? workspace_bytes - abgqa::kWsCounterBytes : 0;
    e = abgqa::launch_attn_prefill(p, st);
  }
  if (log_enabled())
    fprintf(stderr, "[abgqa] attn_bias_gqa_fwd path=%s B=%lld Hq=%lld Hkv=%lld S_q=%lld T=%lld D=%lld D_v=%lld %s splits=%d\n",
            path, (long long)B, (long long)Hq, (long long)Hkv, (long long)S_q, (long long)max_seq,
            (long long)D, (long long)D_v, bias ? "bias" : "rules", p.n_split);
  if (e != hipSuccess) return hip_fail(me, e);
  return chk ? check_after(st, me) : ABGQA_OK;
}

// One fused decode step (attn_decode_step.hip): the checks of kv_scatter_and_bias
// and of attn_bias_gqa_fwd for a shape the split-KV decode kernel takes.
abgqa_status step_impl(const char* me, bool circular, void* out, const void* q, void* k_cache,
                       void* v_cache, const void* k_update, const void* v_update,
                       const int64_t* write_indices, int64_t S_new, void* bias,
                       abgqa_dtype bias_dtype, const int64_t* nonpad_kv_seqlen,
                       const int64_t* q_start, const int32_t* slot_kind, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t S_q, int64_t max_seq, int64_t D, int64_t D_v,
                       float scale, float softcap, int64_t window, abgqa_dtype dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_q <= 0 || max_seq <= 0 || D <= 0 || D_v <= 0)
    return fail(ABGQA_ERR_INVALID, "%s: B, Hq, Hkv, S_q, max_seq, D and D_v must be positive", me);
  if (Hq % Hkv != 0) return fail(ABGQA_ERR_INVALID, "%s: Hq must be a multiple of Hkv", me);
  if (S_new < 0) return fail(ABGQA_ERR_INVALID, "%s: S_new must be >= 0", me);
  if (circular && S_new > max_seq)
    return fail(ABGQA_ERR_INVALID, "%s: a circular cache takes at most capacity = %lld new tokens per call",
                me, (long long)max_seq);
  if (!(softcap >= 0.f) || softcap == INFINITY)
    return fail(ABGQA_ERR_INVALID, "%s: softcap must be finite and >= 0 (0 = none)", me);
  if (S_q > max_seq) return fail(ABGQA_ERR_INVALID, "%s: S_q must not exceed max_seq", me);
  if (max_seq > kMaxSeq) return fail(ABGQA_ERR_UNSUPPORTED, "%s: max_seq above 2^24", me);
  const int64_t G = Hq / Hkv;
  if (dtype != ABGQA_BF16 || S_q * G > 16 || !abgqa::decode_supports((int)D, (int)D_v) ||
      B * Hkv > abgqa::kMaxDecodeRows || S_new > 16)
    return fail(ABGQA_ERR_UNSUPPORTED,
                "%s: the fused step takes bf16 decode shapes (S_q * Hq / Hkv <= 16, D and D_v of the "
                "decode kernel, B * Hkv <= %d, S_new <= 16); use kv_scatter_and_bias and "
                "attn_bias_gqa_fwd", me, (int)abgqa::kMaxDecodeRows);
  if (bias && bias_dtype != ABGQA_F32 && bias_dtype != ABGQA_BF16)
    return fail(ABGQA_ERR_UNSUPPORTED, "%s: bias dtype must be ABGQA_F32 or ABGQA_BF16", me);
  if (!out || !q || !k_cache || !v_cache || !nonpad_kv_seqlen)
    return fail(ABGQA_ERR_INVALID, "%s: null out, q, k_cache, v_cache or nonpad_kv_seqlen", me);
  if (S_new > 0 && (!k_update || !v_update)) return fail(ABGQA_ERR_INVALID, "%s: null update", me);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      (S_new > 0 && (!aligned(k_update, 16) || !aligned(v_update, 16))) ||
      (write_indices && !aligned(write_indices, 8)) || (bias && !aligned(bias, 16)) ||
      !aligned(nonpad_kv_seqlen, 8) || (q_start && !aligned(q_start, 8)) ||
      (slot_kind && !aligned(slot_kind, 16)))
    return fail(ABGQA_ERR_INVALID, "%s: misaligned pointer", me);
  if (out == q || out == k_cache || out == v_cache || out == bias || out == k_update || out == v_update ||
      (bias && (bias == q || bias == k_cache || bias == v_cache)))
    return fail(ABGQA_ERR_INVALID, "%s: out and bias must not alias an input", me);

  abgqa::AttnParams p{};
  p.out = out; p.q = q; p.k = k_cache; p.v = v_cache; p.bias = nullptr;
  p.nonpad = nonpad_kv_seqlen; p.q_start = q_start; p.slot_kind = slot_kind;
  p.B = (int)B; p.Hq = (int)Hq; p.Hkv = (int)Hkv; p.G = (int)G; p.S_q = (int)S_q;
  p.T = (int)max_seq; p.D = (int)D; p.Dv = (int)D_v; p.window = window; p.scale = scale; p.softcap = softcap;
  p.circular = circular ? 1 : 0;
  p.k_upd = k_update; p.v_upd = v_update; p.write_idx = write_indices; p.S_new = (int)S_new;
  p.bias_out = bias; p.bias_out_bf16 = (bias_dtype == ABGQA_BF16);
  hipStream_t st = (hipStream_t)stream;
  const bool chk = check_enabled(st);
  if (chk) {
    abgqa_status r = S_new > 0 ? check_write_indices(write_indices, B, max_seq, S_new, st, me, circular)
                               : ABGQA_OK;
    if (r == ABGQA_OK) r = check_nonpad(nonpad_kv_seqlen, B, max_seq, st, me, circular);
    if (r == ABGQA_OK) r = check_q_start(q_start, B, st, me);
    if (r != ABGQA_OK) return r;
  }
  const abgqa_status r = decode_workspace(me, p, workspace, workspace_bytes, st, chk);
  if (r != ABGQA_OK) return r;
  const hipError_t e = abgqa::launch_decode_step(p, st);
  if (log_enabled())
    fprintf(stderr, "[abgqa] %s B=%lld Hq=%lld Hkv=%lld S_q=%lld S_new=%lld T=%lld D=%lld D_v=%lld splits=%d\n",
            me, (long long)B, (long long)Hq, (long long)Hkv, (long long)S_q, (long long)S_new,
            (long long)max_seq, (long long)D, (long long)D_v, p.n_split);
  if (e != hipSuccess) return hip_fail(me, e);
  return chk ? check_after(st, me) : ABGQA_OK;
}

}  // namespace

extern "C" {

abgqa_status kv_tensor_scatter(void* cache, const void* update, const int64_t* write_indices,
                               int64_t B, int64_t Hkv, int64_t max_seq, int64_t S_new, int64_t D,
                               abgqa_dtype dtype, void* stream) {
  return scatter_impl("kv_tensor_scatter", false, cache, update, write_indices, B, Hkv, max_seq,
                      S_new, D, dtype, stream);
}

abgqa_status kv_tensor_scatter_circular(void* cache, const void* update, const int64_t* write_pos,
                                        int64_t B, int64_t Hkv, int64_t capacity, int64_t S_new,
                                        int64_t D, abgqa_dtype dtype, void* stream) {
  return scatter_impl("kv_tensor_scatter_circular", true, cache, update, write_pos, B, Hkv, capacity,
                      S_new, D, dtype, stream);
}

abgqa_status build_static_cache_bias(void* bias, abgqa_dtype bias_dtype,
                                     const int64_t* nonpad_kv_seqlen, const int64_t* q_start,
                                     const int32_t* slot_kind, int64_t B, int64_t S_q,
                                     int64_t max_seq, int64_t window, void* stream) {
  return bias_impl("build_static_cache_bias", false, bias, bias_dtype, nonpad_kv_seqlen, q_start,
                   slot_kind, B, S_q, max_seq, window, stream);
}

abgqa_status build_circular_cache_bias(void* bias, abgqa_dtype bias_dtype, const int64_t* kv_len,
                                       const int64_t* q_start, const int32_t* slot_kind, int64_t B,
                                       int64_t S_q, int64_t capacity, int64_t window, void* stream) {
  return bias_impl("build_circular_cache_bias", true, bias, bias_dtype, kv_len, q_start, slot_kind, B,
                   S_q, capacity, window, stream);
}

abgqa_status kv_scatter_and_bias(void* k_cache, void* v_cache, const void* k_update,
                                 const void* v_update, const int64_t* write_indices, int64_t B,
                                 int64_t Hkv, int64_t max_seq, int64_t S_new, int64_t D,
                                 abgqa_dtype dtype, void* bias, abgqa_dtype bias_dtype,
                                 const int64_t* nonpad_kv_seqlen, const int64_t* q_start,
                                 const int32_t* slot_kind, int64_t S_q, int64_t window,
                                 void* stream) {
  return prepare_impl("kv_scatter_and_bias", false, k_cache, v_cache, k_update, v_update,
                      write_indices, B, Hkv, max_seq, S_new, D, dtype, bias, bias_dtype,
                      nonpad_kv_seqlen, q_start, slot_kind, S_q, window, stream);
}

abgqa_status kv_scatter_and_bias_circular(void* k_cache, void* v_cache, const void* k_update,
                                          const void* v_update, const int64_t* write_pos, int64_t B,
                                          int64_t Hkv, int64_t capacity, int64_t S_new, int64_t D,
                                          abgqa_dtype dtype, void* bias, abgqa_dtype bias_dtype,
                                          const int64_t* kv_len, const int64_t* q_start,
                                          const int32_t* slot_kind, int64_t S_q, int64_t window,
                                          void* stream) {
  return prepare_impl("kv_scatter_and_bias_circular", true, k_cache, v_cache, k_update, v_update,
                      write_pos, B, Hkv, capacity, S_new, D, dtype, bias, bias_dtype, kv_len, q_start,
                      slot_kind, S_q, window, stream);
}

abgqa_status attn_bias_gqa_fwd(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const void* bias, abgqa_dtype bias_dtype,
                               const int64_t* nonpad_kv_seqlen, const int64_t* q_start,
                               const int32_t* slot_kind, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t S_q, int64_t max_seq, int64_t D, int64_t D_v, float scale,
                               float softcap, int64_t window, abgqa_dtype dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return attn_impl("attn_bias_gqa_fwd", false, out, q, k_cache, v_cache, bias, bias_dtype,
                   nonpad_kv_seqlen, q_start, slot_kind, B, Hq, Hkv, S_q, max_seq, D, D_v, scale,
                   softcap, window, dtype, workspace, workspace_bytes, stream);
}

abgqa_status attn_bias_gqa_fwd_circular(void* out, const void* q, const void* k_cache,
                                        const void* v_cache, const void* bias,
                                        abgqa_dtype bias_dtype, const int64_t* kv_len,
                                        const int64_t* q_start, const int32_t* slot_kind, int64_t B,
                                        int64_t Hq, int64_t Hkv, int64_t S_q, int64_t capacity,
                                        int64_t D, int64_t D_v, float scale, float softcap,
                                        int64_t window, abgqa_dtype dtype, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return attn_impl("attn_bias_gqa_fwd_circular", true, out, q, k_cache, v_cache, bias, bias_dtype,
                   kv_len, q_start, slot_kind, B, Hq, Hkv, S_q, capacity, D, D_v, scale, softcap,
                   window, dtype, workspace, workspace_bytes, stream);
}

abgqa_status attn_bias_gqa_decode_step(void* out, const void* q, void* k_cache, void* v_cache,
                                       const void* k_update, const void* v_update,
                                       const int64_t* write_indices, int64_t S_new, void* bias,
                                       abgqa_dtype bias_dtype, const int64_t* nonpad_kv_seqlen,
                                       const int64_t* q_start, const int32_t* slot_kind, int64_t B,
                                       int64_t Hq, int64_t Hkv, int64_t S_q, int64_t max_seq,
                                       int64_t D, int64_t D_v, float scale, float softcap,
                                       int64_t window, abgqa_dtype dtype, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return step_impl("attn_bias_gqa_decode_step", false, out, q, k_cache, v_cache, k_update, v_update,
                   write_indices, S_new, bias, bias_dtype, nonpad_kv_seqlen, q_start, slot_kind, B, Hq,
                   Hkv, S_q, max_seq, D, D_v, scale, softcap, window, dtype, workspace,
                   workspace_bytes, stream);
}

abgqa_status attn_bias_gqa_decode_step_circular(void* out, const void* q, void* k_cache,
                                                void* v_cache, const void* k_update,
                                                const void* v_update, const int64_t* write_pos,
                                                int64_t S_new, void* bias, abgqa_dtype bias_dtype,
                                                const int64_t* kv_len, const int64_t* q_start,
                                                const int32_t* slot_kind, int64_t B, int64_t Hq,
                                                int64_t Hkv, int64_t S_q, int64_t capacity,
                                                int64_t D, int64_t D_v, float scale, float softcap,
                                                int64_t window, abgqa_dtype dtype, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  return step_impl("attn_bias_gqa_decode_step_circular", true, out, q, k_cache, v_cache, k_update,
                   v_update, write_pos, S_new, bias, bias_dtype, kv_len, q_start, slot_kind, B, Hq,
                   Hkv, S_q, capacity, D, D_v, scale, softcap, window, dtype, workspace,
                   workspace_bytes, stream);
}

const char* abgqa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

// ---------------------------------------------------------------------------
// The entry point that allocates nothing: its scratch is a library-owned
// device array, one per GPU (each device that runs the library holds its own
// copy until the process ends). In host code `scratch` names a host-side
// stand-in, not device memory: only the address hipGetSymbolAddress returns
// for the current device is ever passed to a kernel.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void* ptr = nullptr;   // this device's copy of `scratch`
  bool zeroed = false;   // its arrival counts were cleared by an eager launch
};
std::mutex g_scratch_mu;
DeviceScratch g_scratch[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

extern "C" abgqa_status attn_bias_gqa_fwd_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache, const void* bias,
    abgqa_dtype bias_dtype, const int64_t* nonpad_kv_seqlen, const int64_t* q_start,
    const int32_t* slot_kind, int64_t B, int64_t Hq, int64_t Hkv, int64_t S_q, int64_t max_seq,
    int64_t D, int64_t D_v, float scale, float softcap, int64_t window, abgqa_dtype dtype,
    void* stream) {
  g_last_error.clear();
  const char* me = "attn_bias_gqa_fwd_noalloc";
  const size_t need = attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, max_seq, D, D_v);
  if (need > kNoAllocScratchBytes)
    return fail(ABGQA_ERR_WORKSPACE,
                "%s: this shape needs %zu bytes of scratch; the entry point that allocates nothing "
                "holds %zu per GPU (use attn_bias_gqa_fwd with a workspace)",
                me, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(me, e);
    if (dev < 0 || dev >= kMaxDevices) return fail(ABGQA_ERR_UNSUPPORTED, "%s: device %d beyond %d", me, dev, kMaxDevices);
    const hipStream_t st = (hipStream_t)stream;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    DeviceScratch& ds = g_scratch[dev];
    if (!ds.ptr) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_launch_detail = "hipGetSymbolAddress of the no-alloc scratch";
        return hip_fail(me, e);
      }
      ds.ptr = ptr;
    }
    if (!ds.zeroed) {
      // The decode arrival counts must start at zero (every call leaves them
      // zero). Cleared by a kernel on the caller's stream, not a memset: under
      // graph capture this launch becomes a kernel node, and the device counts
      // as cleared only once an eager call has enqueued it.
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      e = hipStreamIsCapturing(st, &cs);
      if (e != hipSuccess) return hip_fail(me, e);
      constexpr int n = (int)(abgqa::kWsCounterBytes / sizeof(uint32_t));
      hipLaunchKernelGGL(zero_words_kernel, dim3(n / 256), dim3(256), 0, st, (uint32_t*)ds.ptr, n);
      e = hipGetLastError();
      if (e != hipSuccess) {
        g_launch_detail = "no-alloc scratch clear";
        return hip_fail(me, e);
      }
      if (cs == hipStreamCaptureStatusNone) ds.zeroed = true;
    }
    ws = ds.ptr;
  }
  return attn_bias_gqa_fwd(out, q, k_cache, v_cache, bias, bias_dtype, nonpad_kv_seqlen, q_start,
                           slot_kind, B, Hq, Hkv, S_q, max_seq, D, D_v, scale, softcap, window, dtype,
                           ws, ws ? kNoAllocScratchBytes : 0, stream);
}
