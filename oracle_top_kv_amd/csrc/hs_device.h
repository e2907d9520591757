// hs_device.h -- device-side building blocks for gfx950 (CDNA4): MFMA operand types, LDS
// transpose reads, bf16 conversion, order-preserving float keys and wave reductions.
//
// MFMA lane layouts used throughout (wave64, l = lane id):
//   v_mfma_f32_16x16x32_bf16  A[16x32]: lane l holds row l%16, k = 8*(l/16) .. +7
//                             B[32x16]: lane l holds col l%16, k = 8*(l/16) .. +7
//                             C[16x16]: lane l holds col l%16, rows 4*(l/16) .. +3
//   v_mfma_f32_16x16x4_f32    A: row l%16, k = l/16;  B: col l%16, k = l/16;  C as above.
// ds_read_b64_tr_b16 (per 16-lane group): lane r supplies the address of a 4-element row R_r;
// lane i receives { R_{i/4 + 4e}[i%4] : e = 0..3 }.  With lane r pointing at
// tile[kb + r/4][c0 + 4*(r%4)] of a row-major [key][d] tile, lane i receives
// tile[kb + e][c0 + i], e = 0..3: four consecutive keys of one column, which is the MFMA operand
// layout for a contraction over keys.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453;

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS transpose read of four 16-bit elements (see the layout note above).
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) void*)(p)));
}

__device__ __forceinline__ bf16x8 join_tr(const s16x4& lo, const s16x4& hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Eight floats -> bf16x8, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}

// Order-preserving map float -> uint32 (larger float -> larger key; -0 < +0 is fine here).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exchanges between 16-lane rows with the gfx950 swap instructions (VALU, no LDS crossbar).
// v_permlane16_swap(x, x) returns, in each lane, x of that lane and of the same lane in the
// partner row (rows 0<->1, 2<->3); v_permlane32_swap(x, x) does the same for the two halves.
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// max over the 4 lanes {n, n+16, n+32, n+48} (one MFMA row spread over 4 lane groups)
__device__ __forceinline__ float max4groups(float v) { return max_xor32(max_xor16(v)); }

// Lane exchanges inside a 16-lane row with DPP (no LDS crossbar): quad_perm [1,0,3,2] and
// [2,3,0,1], then the half-row and row mirrors.  After the four steps of max16 / min16_u64 every
// lane of the row holds the row's maximum / minimum.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x141>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(dpp_u32<0x140>(__float_as_uint(v))));
}
template <int CTRL>
__device__ __forceinline__ unsigned long long min_dpp_u64(unsigned long long v) {
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)v), hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  return o < v ? o : v;
}
__device__ __forceinline__ unsigned long long min16_u64(unsigned long long v) {
  v = min_dpp_u64<0xB1>(v);
  v = min_dpp_u64<0x4E>(v);
  v = min_dpp_u64<0x141>(v);
  return min_dpp_u64<0x140>(v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Streaming loads for data read once per step (V rows): fetched non-temporally (measured on
// MI355X: about 7.0 TB/s for a pure read stream, against 6.3 TB/s with ordinary loads).  K rows
// use ordinary loads because the selection passes re-read K right after full attention.
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// Kahan-compensated accumulation: the running sum is s - c.
__device__ __forceinline__ void kahan_add(float& s, float& c, float x) {
  const float y = x - c;
  const float t = s + y;
  c = (t - s) - y;
  s = t;
}

// Normalization of one row from its maximum M (log2 domain) and its sum L relative to M, with
// an optional per-head sink logit s (natural log): the softmax denominator becomes
// e^s + sum_i e^a_i, and the sink itself carries no value (the learnable per-head sink bias of
// the pages' sparse and sliding-window layers, P1 section 6.1 and P4 experimental setup, taken
// in the gpt-oss form those pages refer to).  Returns the factor that turns the unnormalized
// output (relative to M) into the output, scaled by `weight`, and the row's LSE including the
// sink.  Without a sink: factor = weight / L and LSE = (M + log2 L) ln 2.
struct RowNorm {
  float factor;
  float lse;
};
__device__ __forceinline__ RowNorm row_norm(float M, double L, const float* sink, int h,
                                            double weight) {
  const double s2 = sink ? (double)sink[h] * 1.4426950408889634 : -INFINITY;
  const double mx = fmax((double)M, s2);
  RowNorm n = {0.f, -INFINITY};
  if (mx == -INFINITY) return n;  // no key and no sink
  const double e = exp2((double)M - mx);  // 1 without a sink; 0 when the row has no key
  const double Lp = L * e + (sink ? exp2(s2 - mx) : 0.0);
  if (!(Lp > 0.0)) return n;
  n.factor = (float)(weight * e / Lp);
  n.lse = (float)((mx + log2(Lp)) * kLn2);
  return n;
}

// Sigmoid output gate of (b, t, h), or 1 without one.
__device__ __forceinline__ double out_gate_of(const float* g, size_t i) {
  return g ? 1.0 / (1.0 + exp(-(double)g[i])) : 1.0;
}

__device__ __forceinline__ float sigmoid_f(float z) {
  return (float)(1.0 / (1.0 + exp(-(double)z)));
}

}  // namespace hs
