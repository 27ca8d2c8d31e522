// Device helpers shared by the gfx950 kernels of libabgqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace abgqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// ---- bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}
// low / high halves of a packed pair of bf16
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (the language cast; gfx950 has a
// native conversion for it).
__device__ __forceinline__ __bf16 f32_to_bf16(float f) { return static_cast<__bf16>(f); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// ---- matrix cores ----------------------------------------------------------
// D[16x16] += A[16x32] * B[32x16], bf16 in, fp32 accumulate.
// Lane l holds A row (l % 16) and B column (l % 16), 8 consecutive k-slots each
// (slots 8*(l/16) .. +7); the result lane l holds column (l % 16), rows
// 4*(l/16) .. +3. Only the pairing of A and B slots matters for a contraction,
// so callers may map the 32 k-slots to any 32 indices as long as A and B agree.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- cross-lane ------------------------------------------------------------
// DPP row (16-lane) controls of the gfx9 family.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// max / sum over the 16 lanes of a DPP row; every lane of the row gets the result
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  return v;
}

// exchange with lane ^ mask. Masks 16 and 32 use the gfx950 lane-swap
// instructions on the vector ALU: v_permlane16_swap / v_permlane32_swap of v
// with itself leave the lower and the upper partner half of each 32- (or
// 64-) lane group in two registers (lane l: v[l & ~m] and v[l | m], checked
// lane by lane on the device), and the lane picks the one that is not its
// own. Other masks go through the LDS crossbar (ds_bpermute, no LDS memory
// used), which queues behind the workgroup's LDS traffic.
__device__ __forceinline__ float lane_xor(float v, int mask) {
  const int lane = __lane_id();
  if (mask == 32 || mask == 16) {
    const unsigned u = __float_as_uint(v);
    const auto r = mask == 32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                              : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((lane & mask) ? r[0] : r[1]);
  }
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, lane_xor(v, 16));
  v = fmaxf(v, lane_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += lane_xor(v, 16);
  v += lane_xor(v, 32);
  return v;
}

// Integer reductions over the 64 lanes of a wavefront, on the vector ALU: DPP
// within each row of 16 lanes, then the 16- and 32-lane swaps (see lane_xor)
// across rows. Every lane gets the result. (Shuffles through the LDS crossbar
// would queue behind the workgroup's LDS traffic.)
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
__device__ __forceinline__ int lane_xor_i32(int v, int mask) {
  return __float_as_int(lane_xor(__int_as_float(v), mask));
}
template <typename Op>
__device__ __forceinline__ int wave_reduce_i32(int v, Op op) {
  v = op(v, dpp_i32<kDppQuadXor1>(v));
  v = op(v, dpp_i32<kDppQuadXor2>(v));
  v = op(v, dpp_i32<kDppRowHalfMirror>(v));
  v = op(v, dpp_i32<kDppRowMirror>(v));
  v = op(v, lane_xor_i32(v, 16));
  v = op(v, lane_xor_i32(v, 32));
  return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
  return wave_reduce_i32(v, [](int a, int b) { return a < b ? a : b; });
}
__device__ __forceinline__ int wave_max_i32(int v) {
  return wave_reduce_i32(v, [](int a, int b) { return a > b ? a : b; });
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  return wave_reduce_i32(v, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ unsigned wave_or_u32(unsigned v) {
  return (unsigned)wave_reduce_i32((int)v, [](int a, int b) { return a | b; });
}
// inclusive prefix sum over the lanes of a wavefront (lane order): within each
// row of 16 by DPP row shifts (lanes shifted in from outside the row add 0),
// then each row adds the totals of the rows before it (read from lanes 15, 31
// and 47)
__device__ __forceinline__ int wave_incl_sum_i32(int v) {
  constexpr int kRowShr = 0x110;   // DPP row_shr:n = 0x110 + n
  v += dpp_i32<kRowShr + 1>(v);
  v += dpp_i32<kRowShr + 2>(v);
  v += dpp_i32<kRowShr + 4>(v);
  v += dpp_i32<kRowShr + 8>(v);
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int lane = __lane_id();
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}
// workgroup barrier for LDS data only: waits for this wavefront's LDS
// accesses, not for its outstanding global loads (__syncthreads waits for both)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// exp2 that maps -inf to exactly 0 (v_exp_f32 does) without NaN for finite input
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(y) = 1 - 2 / (e^(2y) + 1), from the definition: e^(2y) = 2^(2y log2 e)
// on the exponential unit and one hardware reciprocal. The limits are exact
// (2^(2y log2 e) overflows to inf, or underflows to 0, giving +1 or -1); near 0
// the error is a few units in the last place of 1.
__device__ __forceinline__ float fast_tanh(float y) {
  return 1.f - 2.f * __builtin_amdgcn_rcpf(1.f + fast_exp2(y * (2.f * kLog2e)));
}

// The softcap stage on base-2 scores t = scale * q.k * log2(e): c * tanh(v / c)
// in natural units is (c log2 e) * tanh(t / (c log2 e)) in base 2, i.e.
// cap2 * tanh(raw * (scale / c)) for the raw dot product `raw`.
__device__ __forceinline__ float softcap_base2(float raw, float cap2, float scale_over_cap) {
  return cap2 * fast_tanh(raw * scale_over_cap);
}

// ---- grid mapping ----------------------------------------------------------
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with its own L2. Remap so that consecutive logical ids run on one XCD (and
// share its L2): hardware id h -> logical (h % 8) * ceil(n/8) + h / 8, with the
// ids past n (when n % 8 != 0) folded back in order.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_remap(int hw, int n) {
  const int per = (n + kNumXcd - 1) / kNumXcd;
  const int full = n - (per - 1) * kNumXcd;  // XCDs that get `per` ids
  const int xcd = hw % kNumXcd;
  const int idx = hw / kNumXcd;
  return (xcd < full) ? xcd * per + idx : full * per + (xcd - full) * (per - 1) + idx;
}

// ---- memory ----------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
  return *reinterpret_cast<const T*>(p);
}
// A load of data that is read once (the K and V rows a decode call streams):
// non-temporal, so the lines are not kept in the caches for reuse that will
// not come, and do not push out what will be reused.
template <typename T>
__device__ __forceinline__ T ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}
// A store of data that is not read again by this call (the prefill output
// rows): non-temporal, so it does not push the K/V tiles that the other query
// tiles still fetch out of the caches.
template <typename T>
__device__ __forceinline__ void st_stream(void* p, const T& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
}

__device__ __forceinline__ int64_t clamp_nonpad(int64_t np, int64_t max_seq) {
  return np < 0 ? 0 : (np > max_seq ? max_seq : np);
}

}  // namespace abgqa
