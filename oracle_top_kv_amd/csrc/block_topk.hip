// block_topk.hip -- HySparse block-level oracle index [P2 "Extracting block scores from exact
// attention", block-score and TopK equations; P2 "GQA: the group shares one index set";
// P4 section 3.2 and Algorithm 1, whose normalization of the block maximum needs the
// exponential that the printed algorithm leaves out, as P2 points out].
//
// Block score of causal block r for query row (b, t, u):
//   S_r = max_{h in group u} max_{i in [rB, min(rB+B-1, t)]} exp(a^h_{t,i} - LSE^h_t),
// ranked in the log2 domain as max(a * log2(e) - (LSE * log2(e) - C)) like the token scores.
// The logits are recomputed (MFMA, S = Q K^T) rather than stored per tile, so no T x T/B score
// matrix exists anywhere.
//
// Two kernels:
//   1. per (key split, row-set): every block of the split is scored; the split's exact top-n
//      blocks per query (n = n_blocks) are written as 64-bit keys (score key << 32 | ~block id),
//      so larger key = better and equal scores prefer the lower block id;
//   2. per query row: the top-n of the union of the splits' candidates (exact: the global top-n
//      is contained in the union of per-split top-n), written in ascending block order.
#include "hs_device.h"
#include "hs_kernels.h"
#include "score_common.h"

namespace hs {
namespace {

constexpr int kMaxRange = 256;  // blocks per split (per workgroup)

template <int D, bool F32>
__global__ __launch_bounds__(256) void blk_score_kernel(BlockTopkParams p) {
  __shared__ unsigned long long bkey[4][kMaxRange];  // per query of the set, per block of the split
  __shared__ uint32_t bmax[4][kMaxRange];             // running block maxima (order-preserving keys)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rn = lane & 15, jg = lane >> 4;
  // KV head fastest, then split, then (batch, query chunk): see the row-attention kernel
  const int u = blockIdx.x % p.Hkv;
  const int split = (blockIdx.x / p.Hkv) % p.n_split;
  const int bq = blockIdx.x / (p.Hkv * p.n_split);
  const int sq = bq % p.sets_per_bu;
  const int b = bq / p.sets_per_bu;
  const int j0 = sq * p.q_per_set;
  const int nq = min(p.q_per_set, p.Tq - j0);
  const int nrows = nq * p.g;
  const int G = p.g / 4;

  const long long blk_begin = (long long)split * p.blocks_per_split;
  const long long t_last = p.q_off + j0 + nq - 1;
  long long blk_end = blk_begin + p.blocks_per_split;
  if (blk_end > t_last / p.block + 1) blk_end = t_last / p.block + 1;
  const int n_range = blk_end > blk_begin ? (int)(blk_end - blk_begin) : 0;
  for (int i = threadIdx.x; i < 4 * kMaxRange; i += 256) {
    (&bkey[0][0])[i] = 0ull;
    (&bmax[0][0])[i] = 0u;
  }

  constexpr int KK = KTile<D, F32>::KK;
  const bool row_ok = rn < nrows;
  const int jq_r = row_ok ? rn / p.g : 0, hh_r = row_ok ? rn % p.g : 0;
  bf16x8 qa[F32 ? 1 : KK];
  float qf[F32 ? KK : 1];
  {
    const size_t qoff = (((size_t)b * p.Tq + j0 + jq_r) * p.Hq + u * p.g + hh_r) * D;
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
      for (int s = 0; s < KK; s++) qf[s] = row_ok ? qp[s] : 0.f;
    }
  }
  float delta[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int r = 4 * jg + e;
    if (r < nrows) {
      const int j = j0 + r / p.g, hh = r % p.g;
      const double l2 = (double)p.lse[((size_t)b * p.Hq + u * p.g + hh) * p.Tq + j] * 1.4426950408889634;
      const double C = rint((double)p.lse[((size_t)b * p.Hq + u * p.g) * p.Tq + j] * 1.4426950408889634);
      delta[e] = (float)(l2 - C);
    } else {
      delta[e] = INFINITY;
    }
  }
  const int jq_own = jg / G;
  const bool owner = (jg % G) == 0 && jq_own < nq;
  const long long t_own = p.q_off + j0 + jq_own;
  __syncthreads();

  const size_t kv_row_stride = (size_t)p.Hkv * D;
  const size_t kv_base = ((size_t)b * p.Tk * p.Hkv + u) * D;
  // keys of this split's blocks, in 64-key tiles interleaved over the waves; every 16-key
  // group's maximum is folded into its block with an LDS atomicMax on order-preserving keys
  const long long key_begin = blk_begin * p.block;
  long long key_end = blk_end * p.block;
  if (key_end > t_last + 1) key_end = t_last + 1;
  // one 64-key tile already in registers
  auto score_tile = [&](const KTile<D, F32>& cur, long long tile) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const long long g0 = tile + 16 * kb;  // first key of the group
      const long long pos = g0 + rn;
      const f32x4 acc = score_block<D, F32>(cur, kb, qa, qf);
      float v = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; e++) v = fmaxf(v, __builtin_fmaf(acc[e], p.scale_log2, -delta[e]));
      if (G >= 2) v = max_xor16(v);
      if (G >= 4) v = max_xor32(v);
      // causal: keys after this lane's query position do not count
      if (pos > t_own || pos >= key_end) v = -INFINITY;
      // max over the 16 keys of the group (lanes of one 16-lane row)
      v = max16(v);
      const long long blk = g0 / p.block;
      if (owner && rn == 0 && g0 < key_end && g0 <= t_own)
        atomicMax(&bmax[jq_own][blk - blk_begin], float_key(v));
    }
  };
  // The loop always prefetches the next tile (the last tile is peeled off): with a conditional
  // prefetch the compiler waits for the prefetched loads before computing each tile.
  KTile<D, F32> cur, nxt;
  long long tile = key_begin + 64LL * wave;
  if (tile < key_end) load_k_tile<D, F32>(cur, p.k, kv_base, kv_row_stride, tile, p.Tk, rn, jg);
  for (; tile + 256 < key_end; tile += 64LL * 4) {
    load_k_tile<D, F32>(nxt, p.k, kv_base, kv_row_stride, tile + 256, p.Tk, rn, jg);
    score_tile(cur, tile);
    cur = nxt;
  }
  if (tile < key_end) score_tile(cur, tile);
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * n_range; i += 256) {
    const int jq = i / n_range, rb = i % n_range;
    const long long blk = blk_begin + rb;
    if (jq < nq && blk <= (p.q_off + j0 + jq) / p.block)
      bkey[jq][rb] = ((unsigned long long)bmax[jq][rb] << 32) |
                     (unsigned long long)(0xFFFFFFFFu - (uint32_t)blk);
  }
  __syncthreads();
  // exact local top-n per query: rank = number of strictly larger keys (keys are distinct)
  for (int jq = 0; jq < nq; jq++) {
    const long long row = ((long long)b * p.Tq + j0 + jq) * p.Hkv + u;
    unsigned long long* out = p.cand + ((size_t)row * p.n_split + split) * p.n_blocks;
    for (int c = threadIdx.x; c < n_range; c += 256) {
      const unsigned long long kc = bkey[jq][c];
      if (kc == 0ull) continue;
      int rank = 0;
      for (int o = 0; o < n_range; o++) rank += bkey[jq][o] > kc;
      if (rank < p.n_blocks) out[rank] = kc;
    }
    // fill the unused slots with 0 (no candidate)
    int valid = 0;
    for (int c = 0; c < n_range; c++) valid += bkey[jq][c] != 0ull;
    for (int s = valid + threadIdx.x; s < p.n_blocks; s += 256) out[s] = 0ull;
  }
}

// Block scores from the raw dot products q.k that the full-attention pass stored
// ([B, Tq, Hq, Tk] fp32): same key and same local top-n as blk_score_kernel, without reading Q
// or K.  One workgroup per (row, block split); a thread per key, a 16-lane row per 16 keys.
template <int G>
__global__ __launch_bounds__(256) void blk_logit_score_kernel(BlockTopkParams p) {
  __shared__ unsigned long long bkey[kMaxRange];
  __shared__ uint32_t bmax[kMaxRange];
  __shared__ float dsh[64];
  const int split = blockIdx.x % p.n_split;
  const int row = blockIdx.x / p.n_split;  // (b * Tq + j) * Hkv + u
  const int u = row % p.Hkv;
  const int j = (row / p.Hkv) % p.Tq;
  const int b = row / (p.Hkv * p.Tq);
  const long long t = p.q_off + j;
  const long long blk_begin = (long long)split * p.blocks_per_split;
  long long blk_end = blk_begin + p.blocks_per_split;
  if (blk_end > t / p.block + 1) blk_end = t / p.block + 1;
  const int n_range = blk_end > blk_begin ? (int)(blk_end - blk_begin) : 0;
  for (int i = threadIdx.x; i < kMaxRange; i += 256) {
    bkey[i] = 0ull;
    bmax[i] = 0u;
  }
  if (threadIdx.x < G) {
    // per-head shift LSE_h * log2(e) - C, C from the group's first head (as in the score pass);
    // heads past the group's g (G is the instantiated bound) never score
    const int hh = threadIdx.x;
    const double l2 = hh < p.g ? (double)p.lse[((size_t)b * p.Hq + u * p.g + hh) * p.Tq + j] * 1.4426950408889634 : 0.0;
    const double C = rint((double)p.lse[((size_t)b * p.Hq + u * p.g) * p.Tq + j] * 1.4426950408889634);
    dsh[threadIdx.x] = hh < p.g ? (float)(l2 - C) : INFINITY;
  }
  __syncthreads();
  float delta[G];
#pragma unroll
  for (int hh = 0; hh < G; hh++) delta[hh] = dsh[hh];
  const long long key_begin = blk_begin * p.block;  // a multiple of 16
  long long key_end = blk_end * p.block;
  if (key_end > t + 1) key_end = t + 1;
  const float* lg = p.logits + (((size_t)b * p.Tq + j) * p.Hq + (size_t)u * p.g) * p.Tk;
  for (long long base = key_begin; base < key_end; base += 256) {
    const long long pos = base + threadIdx.x;
    float v = -INFINITY;
    if (pos < key_end) {
      float x[G];
#pragma unroll
      for (int hh = 0; hh < G; hh++) x[hh] = hh < p.g ? lg[(size_t)hh * p.Tk + pos] : 0.f;
#pragma unroll
      for (int hh = 0; hh < G; hh++) v = fmaxf(v, __builtin_fmaf(x[hh], p.scale_log2, -delta[hh]));
    }
    // max over the 16 keys of this lane row (they lie in one block: block % 16 == 0)
    v = max16(v);
    if ((threadIdx.x & 15) == 0 && pos < key_end)
      atomicMax(&bmax[pos / p.block - blk_begin], float_key(v));
  }
  __syncthreads();
  for (int rb = threadIdx.x; rb < n_range; rb += 256)
    bkey[rb] = ((unsigned long long)bmax[rb] << 32) |
               (unsigned long long)(0xFFFFFFFFu - (uint32_t)(blk_begin + rb));
  __syncthreads();
  unsigned long long* out = p.cand + ((size_t)row * p.n_split + split) * p.n_blocks;
  for (int c = threadIdx.x; c < n_range; c += 256) {
    const unsigned long long kc = bkey[c];
    int rank = 0;
    for (int o = 0; o < n_range; o++) rank += bkey[o] > kc;
    if (rank < p.n_blocks) out[rank] = kc;
  }
  for (int s = n_range + threadIdx.x; s < p.n_blocks; s += 256) out[s] = 0ull;
}

__global__ __launch_bounds__(256) void blk_merge_kernel(BlockTopkParams p) {
  extern __shared__ unsigned long long cand[];  // n_split * n_blocks
  __shared__ int sel_ids[64];
  const int row = blockIdx.x;
  const int j = (row / p.Hkv) % p.Tq;
  const long long t = p.q_off + j;
  const long long nb = t / p.block + 1;
  const int n_take = (int)(nb < p.n_blocks ? nb : p.n_blocks);
  const int R = p.n_split * p.n_blocks;
  const unsigned long long* src = p.cand + (size_t)row * R;
  for (int i = threadIdx.x; i < R; i += 256) cand[i] = src[i];
  __syncthreads();
  for (int c = threadIdx.x; c < R; c += 256) {
    const unsigned long long kc = cand[c];
    if (kc == 0ull) continue;
    int rank = 0;
    for (int o = 0; o < R; o++) rank += cand[o] > kc;
    if (rank < n_take) sel_ids[rank] = (int)(0xFFFFFFFFu - (uint32_t)(kc & 0xFFFFFFFFull));
  }
  __syncthreads();
  // ascending block ids
  int32_t* out = p.blk_idx + (size_t)row * p.n_blocks;
  for (int s = threadIdx.x; s < p.n_blocks; s += 256) {
    if (s < n_take) {
      const int id = sel_ids[s];
      int pos = 0;
      for (int o = 0; o < n_take; o++) pos += sel_ids[o] < id;
      out[pos] = id;
    } else {
      out[s] = -1;
    }
  }
  if (threadIdx.x == 0) p.cnt[row] = n_take;
}

template <int D, bool F32>
hipError_t launch_blk(const BlockTopkParams& p, hipStream_t stream) {
  blk_score_kernel<D, F32><<<dim3(p.n_split * p.B * p.Hkv * p.sets_per_bu), 256, 0, stream>>>(p);
  const size_t rows = (size_t)p.B * p.Tq * p.Hkv;
  const size_t smem = (size_t)p.n_split * p.n_blocks * sizeof(unsigned long long);
  blk_merge_kernel<<<dim3((unsigned)rows), 256, smem, stream>>>(p);
  return hipGetLastError();
}

template <int G>
hipError_t launch_blk_logits(const BlockTopkParams& p, hipStream_t stream) {
  const size_t rows = (size_t)p.B * p.Tq * p.Hkv;
  blk_logit_score_kernel<G><<<dim3((unsigned)(p.n_split * rows)), 256, 0, stream>>>(p);
  const size_t smem = (size_t)p.n_split * p.n_blocks * sizeof(unsigned long long);
  blk_merge_kernel<<<dim3((unsigned)rows), 256, smem, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_from_logits(const BlockTopkParams& p, hipStream_t stream) {
  switch (p.g) {
    case 1: return launch_blk_logits<1>(p, stream);
    case 2: return launch_blk_logits<2>(p, stream);
    case 3: return launch_blk_logits<3>(p, stream);
    case 4: return launch_blk_logits<4>(p, stream);
    case 5: return launch_blk_logits<5>(p, stream);
    case 6: return launch_blk_logits<6>(p, stream);
    case 7: return launch_blk_logits<7>(p, stream);
    case 8: return launch_blk_logits<8>(p, stream);
    case 9: return launch_blk_logits<9>(p, stream);
    case 10: return launch_blk_logits<10>(p, stream);
    case 11: return launch_blk_logits<11>(p, stream);
    case 12: return launch_blk_logits<12>(p, stream);
    case 13: return launch_blk_logits<13>(p, stream);
    case 14: return launch_blk_logits<14>(p, stream);
    case 15: return launch_blk_logits<15>(p, stream);
    case 16: return launch_blk_logits<16>(p, stream);
    case 32: return launch_blk_logits<32>(p, stream);
    case 48: return launch_blk_logits<48>(p, stream);
    case 64: return launch_blk_logits<64>(p, stream);
  }
  // other group sizes run on the next larger instantiation, the extra heads masked
  if (p.g < 32) return launch_blk_logits<32>(p, stream);
  if (p.g < 48) return launch_blk_logits<48>(p, stream);
  if (p.g < 64) return launch_blk_logits<64>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_block_topk(const BlockTopkParams& p, int head_dim, bool in_f32,
                             hipStream_t stream) {
  if (head_dim == 128) return in_f32 ? launch_blk<128, true>(p, stream) : launch_blk<128, false>(p, stream);
  return in_f32 ? launch_blk<64, true>(p, stream) : launch_blk<64, false>(p, stream);
}

}  // namespace hs
