// logits.hip -- raw attention logits q.k of few query rows over their whole causal key range,
// for the index selection of shapes the fused score passes do not cover (GQA groups other than
// 4, 8 or 16 heads, head size 256): the selection then ranks these values exactly as it ranks
// the logits a full-attention pass keeps [P2 "Why normalize scores for TopK" and "Extracting
// block scores from exact attention": the normalized scores may come from a second pass once
// the LSE is known].
//
// S = Q K^T on MFMA, 16 query heads of one (batch entry, query, KV head) per wave (a chunk of the
// group; the last chunk of a group that is not a multiple of 16 has rows without a head), K read
// straight from HBM in 64-key tiles (score_common.h).  Output [B, Tq, Hq, Tk] fp32, entries
// 0..t of query row t (before the 1/sqrt(d) scale).
#include "hs_device.h"
#include "hs_kernels.h"
#include "score_common.h"

namespace hs {
namespace {

template <int D, bool F32>
__global__ __launch_bounds__(256) void logits_kernel(LogitsParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rn = lane & 15, jg = lane >> 4;
  const int n_chunks = (p.g + 15) / 16;
  // workgroup -> (batch, query, KV head, chunk, key split), split fastest
  const int split = blockIdx.x % p.n_split;
  int rest = blockIdx.x / p.n_split;
  const int c = rest % n_chunks;
  rest /= n_chunks;
  const int u = rest % p.Hkv;
  rest /= p.Hkv;
  const int j = rest % p.Tq;
  const int b = rest / p.Tq;
  const long long t = p.q_off + j;

  constexpr int KK = KTile<D, F32>::KK;
  const bool row_ok = c * 16 + rn < p.g;
  const int h_row = u * p.g + c * 16 + (row_ok ? rn : 0);
  bf16x8 qa[F32 ? 1 : KK];
  float qf[F32 ? KK : 1];
  {
    const size_t qoff = (((size_t)b * p.Tq + j) * p.Hq + h_row) * D;
    if constexpr (!F32) {
      const uint16_t* qp = (const uint16_t*)p.q + qoff;
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        u32x4 raw = row_ok ? *(const u32x4*)(qp + 32 * kk + 8 * jg) : u32x4{0, 0, 0, 0};
        qa[kk] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
      const float* qp = (const float*)p.q + qoff + jg * KK;
#pragma unroll
      for (int s2 = 0; s2 < KK; s2++) qf[s2] = row_ok ? qp[s2] : 0.f;
    }
  }
  // output rows of this lane: heads c * 16 + 4 jg + e
  float* out[4];
  bool out_ok[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int hh = c * 16 + 4 * jg + e;
    out_ok[e] = hh < p.g;
    out[e] = p.logits + (((size_t)b * p.Tq + j) * p.Hq + u * p.g + (out_ok[e] ? hh : 0)) * (size_t)p.Tk;
  }
  const size_t kv_row_stride = (size_t)p.Hkv * D;
  const size_t kv_base = ((size_t)b * p.Tk * p.Hkv + u) * D;
  const long long k_begin = (long long)split * p.keys_per_split;
  long long k_end = k_begin + p.keys_per_split;
  if (k_end > t + 1) k_end = t + 1;
  for (long long tile = k_begin + 64LL * wave; tile < k_end; tile += 256) {
    KTile<D, F32> kt;
    load_k_tile<D, F32>(kt, p.k, kv_base, kv_row_stride, tile, p.Tk, rn, jg);
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const f32x4 acc = score_block<D, F32>(kt, kb, qa, qf);
      const long long pos = tile + 16 * kb + rn;
      if (pos < k_end) {
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (out_ok[e]) out[e][pos] = acc[e];
      }
    }
  }
}

}  // namespace

hipError_t launch_logits(const LogitsParams& p, int head_dim, bool in_f32, hipStream_t stream) {
  const int n_chunks = (p.g + 15) / 16;
  const dim3 grid((unsigned)((long long)p.B * p.Tq * p.Hkv * n_chunks * p.n_split));
  if (p.keys_per_split % 256) return hipErrorInvalidValue;
  if (head_dim == 256) {
    if (in_f32) return hipErrorInvalidValue;
    logits_kernel<256, false><<<grid, 256, 0, stream>>>(p);
  } else if (head_dim == 128) {
    if (in_f32) logits_kernel<128, true><<<grid, 256, 0, stream>>>(p);
    else logits_kernel<128, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (in_f32) logits_kernel<64, true><<<grid, 256, 0, stream>>>(p);
    else logits_kernel<64, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace hs
