// score_common.h -- shared by the token and block score passes: Q rows as the MFMA A operand,
// a 64-key tile of K as four B operands (S = Q K^T, so the g head values of one key sit in one
// lane or one lane row), loaded one tile ahead of its use.  K is loaded with ordinary (cached)
// loads: the score pass runs right after the full-attention pass over the same K, and part of
// it is still in the last-level cache.
#pragma once
#include <type_traits>

#include "hs_device.h"

namespace hs {

template <int D, bool F32>
struct KTile {
  static constexpr int KK = F32 ? D / 4 : D / 32;  // MFMA steps over d
  using R = typename std::conditional<F32, float, u32x4>::type;
  R r[4][KK];
};

// Lane (key rn, group jg) loads, for each 16-key block kb of the tile starting at `tile`, the
// part of row tile + 16 kb + rn that the MFMA B operand needs (rows past the end read row 0).
template <int D, bool F32>
__device__ __forceinline__ void load_k_tile(KTile<D, F32>& t, const void* k, size_t kv_base,
                                            size_t row_stride, long long tile, long long n_rows,
                                            int rn, int jg) {
  constexpr int KK = KTile<D, F32>::KK;
#pragma unroll
  for (int kb = 0; kb < 4; kb++) {
    const long long pos = tile + 16 * kb + rn;
    const size_t pc = (size_t)(pos < n_rows ? pos : 0);
    if constexpr (!F32) {
      const uint16_t* kp = (const uint16_t*)k + kv_base + pc * row_stride + 8 * jg;
#pragma unroll
      for (int kk = 0; kk < KK; kk++) t.r[kb][kk] = *(const u32x4*)(kp + 32 * kk);
    } else {
      const float* kp = (const float*)k + kv_base + pc * row_stride + jg * KK;
#pragma unroll
      for (int s = 0; s < KK; s++) t.r[kb][s] = kp[s];
    }
  }
}

// S block (16 rows x 16 keys) of key block kb: lane (key rn, group jg) gets rows 4jg..4jg+3.
template <int D, bool F32>
__device__ __forceinline__ f32x4 score_block(const KTile<D, F32>& t, int kb, const bf16x8* qa,
                                             const float* qf) {
  constexpr int KK = KTile<D, F32>::KK;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!F32) {
#pragma unroll
    for (int kk = 0; kk < KK; kk++) acc = mfma_bf16(qa[kk], __builtin_bit_cast(bf16x8, t.r[kb][kk]), acc);
  } else {
#pragma unroll
    for (int s = 0; s < KK; s++) acc = mfma_f32(qf[s], t.r[kb][s], acc);
  }
  return acc;
}

}  // namespace hs
