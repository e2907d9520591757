// topk_decode.hip -- exact token top-k for few query rows per KV head over long contexts
// (decode), the HySparse2 oracle index [P1 section 4.2 changes 1 and 2; P5 "KV Reuse (Inner
// Level)"].
//
// Score of key i for query row (b, t, u): s_i = max_{h in group u} p^h_{t,i} with
// p = exp(a - LSE) [P2 "Extracting block scores from exact attention"; P2 "GQA: the group shares
// one index set"].  It is ranked in the log2 domain as
//     key_i = max_h ( a^h_i * log2(e) - (LSE^h * log2(e) - C) ),   C = per-row integer constant,
// which orders exactly like p (a per-row shift; the constant keeps the fp32 values small so the
// representation error stays near 1e-7).  Only positions 0..t-w are candidates; the w most
// recent positions are always taken.
//
// Pipeline (one row = one (b, t, u)):
//   1. score: recompute the logits (MFMA, S = Q K^T so a key's g head values sit in one lane or
//      one lane row), write the order-preserving 32-bit key per candidate and a histogram of its
//      top 11 bits;
//   2. radix passes on bits 20..10 and 9..0 among the keys that match the prefix found so far;
//   3. the exact k-th key value T and how many keys equal to T are taken (lowest positions
//      first: the tie rule is position ascending);
//   4. ordered compaction per chunk (keys > T, and the first keys == T) into the index list,
//      which is therefore ascending; the window positions follow; -1 padding to the cap.
// All steps are exact: nothing is dropped by an approximation.
#include "hs_device.h"
#include "hs_kernels.h"

namespace hs {
namespace {

constexpr int kBins = 2048;

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---- 1. score + first histogram ----------------------------------------------------------
template <int D, bool F32>
__global__ __launch_bounds__(256) void tk_score_kernel(TopkDecodeParams p) {
  __shared__ uint32_t hist[4][kBins];  // one per query row of the set (q_per_set * g <= 16, g >= 4)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rn = lane & 15, jg = lane >> 4;
  const int split = blockIdx.x;
  const int set = blockIdx.y;
  const int sq = set % p.sets_per_bu;
  const int bu = set / p.sets_per_bu;
  const int u = bu % p.Hkv, b = bu / p.Hkv;
  const int j0 = sq * p.q_per_set;
  const int nq = min(p.q_per_set, p.Tq - j0);
  const int nrows = nq * p.g;
  const int G = p.g / 4;  // lane groups per query

  for (int i = threadIdx.x; i < 4 * kBins; i += 256) (&hist[0][0])[i] = 0u;

  // A operand: Q rows (row r = jq * g + hh)
  constexpr int KK = F32 ? D / 4 : D / 32;  // MFMA steps over d
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
  // per-row shift delta_r = LSE_r * log2(e) - C_jq, in double then rounded (|delta| is small)
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
      delta[e] = INFINITY;  // padding rows never win the max
    }
  }
  // the query this lane's group reports for, and its last candidate position
  const int jq_own = jg / G;
  const bool owner = (jg % G) == 0 && jq_own < nq;
  const long long t_own = p.q_off + j0 + jq_own;
  const long long last_cand = t_own - p.window;  // candidates 0 .. t - w
  const long long row_own = ((long long)b * p.Tq + j0 + jq_own) * p.Hkv + u;
  uint32_t* keys_row = p.keys + (size_t)(owner ? row_own : 0) * p.Tk;
  __syncthreads();

  const long long max_cand = p.q_off + j0 + nq - 1 - p.window;  // over the set's queries
  const long long k_begin = (long long)split * p.keys_per_split;
  long long k_end = k_begin + p.keys_per_split;
  if (k_end > max_cand + 1) k_end = max_cand + 1;
  const size_t kv_row_stride = (size_t)p.Hkv * D;
  const size_t kv_base = ((size_t)b * p.Tk * p.Hkv + u) * D;

  for (long long tile = k_begin + 64LL * wave; tile < k_end; tile += 64LL * 4) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const long long pos = tile + 16 * kb + rn;
      const long long pc = pos < p.Tk ? pos : 0;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!F32) {
        const uint16_t* kp = (const uint16_t*)p.k + kv_base + (size_t)pc * kv_row_stride;
#pragma unroll
        for (int kk = 0; kk < KK; kk++) {
          u32x4 raw = *(const u32x4*)(kp + 32 * kk + 8 * jg);
          acc = mfma_bf16(qa[kk], __builtin_bit_cast(bf16x8, raw), acc);
        }
      } else {
        const float* kp = (const float*)p.k + kv_base + (size_t)pc * kv_row_stride + jg * KK;
#pragma unroll
        for (int s = 0; s < KK; s++) acc = mfma_f32(qf[s], kp[s], acc);
      }
      // lane (key rn, group jg) holds rows 4jg..4jg+3 for key `pos`
      float v = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; e++) v = fmaxf(v, __builtin_fmaf(acc[e], p.scale_log2, -delta[e]));
      if (G >= 2) v = fmaxf(v, __shfl_xor(v, 16, 64));
      if (G >= 4) v = fmaxf(v, __shfl_xor(v, 32, 64));
      if (owner && pos <= last_cand && pos < k_end) {
        const uint32_t key = float_key(v);
        keys_row[pos] = key;
        atomicAdd(&hist[jq_own][key >> 21], 1u);
      }
    }
  }
  __syncthreads();
  for (int jq = 0; jq < nq; jq++) {
    uint32_t* gh = p.hist + ((size_t)((b * p.Tq + j0 + jq) * p.Hkv + u)) * kBins;
    for (int i = threadIdx.x; i < kBins; i += 256) {
      const uint32_t c = hist[jq][i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

// Find, scanning bins from the top, the bin holding the k-th largest element; returns the bin
// and the rank k' of that element within the bin (1-based).  All 256 threads call it.
__device__ void find_bin(const uint32_t* h, int k, int* bin_out, int* k_out) {
  __shared__ uint32_t part[256];
  // thread i owns bins [8*(255-i), 8*(255-i)+8): thread 0 owns the top bins
  const int base = 8 * (255 - threadIdx.x);
  uint32_t s = 0;
#pragma unroll
  for (int q = 0; q < 8; q++) s += h[base + q];
  part[threadIdx.x] = s;
  __syncthreads();
  // inclusive prefix over threads (top-down order) by a simple log-step scan
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t x = threadIdx.x >= off ? part[threadIdx.x - off] : 0u;
    __syncthreads();
    part[threadIdx.x] += x;
    __syncthreads();
  }
  const uint32_t incl = part[threadIdx.x];
  const uint32_t excl = incl - s;
  if ((int)excl < k && k <= (int)incl) {
    uint32_t cum = excl;
    for (int q = 7; q >= 0; q--) {
      const uint32_t c = h[base + q];
      if ((int)(cum + c) >= k) {
        *bin_out = base + q;
        *k_out = k - (int)cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

struct RowSel {
  int k_eff;  // number of candidates to take
  long long n_cand;
  long long t;
};

__device__ __forceinline__ RowSel row_sel(const TopkDecodeParams& p, int row) {
  const int j = (row / p.Hkv) % p.Tq;
  RowSel r;
  r.t = p.q_off + j;
  r.n_cand = r.t - p.window + 1;
  if (r.n_cand < 0) r.n_cand = 0;
  r.k_eff = (int)(r.n_cand < p.k_global ? r.n_cand : p.k_global);
  return r;
}

// ---- 2. radix passes on the lower digits ---------------------------------------------------
// PASS 1: digit bits 20..10 among keys whose bits 31..21 match; PASS 2: bits 9..0.
template <int PASS>
__global__ __launch_bounds__(256) void tk_pass_kernel(TopkDecodeParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ int sel[4];
  const int split = blockIdx.x, row = blockIdx.y;
  if (threadIdx.x < 4) sel[threadIdx.x] = 0;
  const RowSel rs = row_sel(p, row);
  if (rs.k_eff == 0) return;
  const size_t nrows = (size_t)p.B * p.Tq * p.Hkv;
  const uint32_t* h0 = p.hist + (size_t)row * kBins;
  const uint32_t* h1 = p.hist + (nrows + row) * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = 0u;
  find_bin(h0, rs.k_eff, &sel[0], &sel[1]);
  if (PASS == 2) find_bin(h1, sel[1], &sel[2], &sel[3]);
  __syncthreads();
  const uint32_t b1 = sel[0];
  const uint32_t b2 = PASS == 2 ? (uint32_t)sel[2] : 0u;
  const long long k_begin = (long long)split * p.keys_per_split;
  long long k_end = k_begin + p.keys_per_split;
  if (k_end > rs.n_cand) k_end = rs.n_cand;
  const uint32_t* keys = p.keys + (size_t)row * p.Tk;
  for (long long i = k_begin + threadIdx.x; i < k_end; i += 256) {
    const uint32_t key = keys[i];
    if ((key >> 21) != b1) continue;
    if (PASS == 1) {
      atomicAdd(&hist[(key >> 10) & 2047u], 1u);
    } else if (((key >> 10) & 2047u) == b2) {
      atomicAdd(&hist[key & 1023u], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = p.hist + ((PASS == 1 ? nrows : 2 * nrows) + row) * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// ---- 3. exact threshold, per-chunk counts ------------------------------------------------
__device__ void threshold(const TopkDecodeParams& p, int row, int k_eff, uint32_t* T, int* k_eq) {
  __shared__ int sel[6];
  const size_t nrows = (size_t)p.B * p.Tq * p.Hkv;
  if (threadIdx.x < 6) sel[threadIdx.x] = 0;
  __syncthreads();
  find_bin(p.hist + (size_t)row * kBins, k_eff, &sel[0], &sel[1]);
  find_bin(p.hist + (nrows + row) * kBins, sel[1], &sel[2], &sel[3]);
  find_bin(p.hist + (2 * nrows + row) * kBins, sel[3], &sel[4], &sel[5]);
  __syncthreads();
  *T = ((uint32_t)sel[0] << 21) | ((uint32_t)sel[2] << 10) | (uint32_t)sel[4];
  *k_eq = sel[5];
}

__global__ __launch_bounds__(256) void tk_count_kernel(TopkDecodeParams p) {
  __shared__ uint32_t tot[2];
  const int split = blockIdx.x, row = blockIdx.y;
  const RowSel rs = row_sel(p, row);
  uint32_t* cnt = p.counts + ((size_t)row * p.n_split + split) * 2;
  if (rs.k_eff == 0) {
    if (threadIdx.x == 0) cnt[0] = cnt[1] = 0u;
    return;
  }
  uint32_t T;
  int k_eq;
  threshold(p, row, rs.k_eff, &T, &k_eq);
  if (threadIdx.x < 2) tot[threadIdx.x] = 0u;
  __syncthreads();
  const long long k_begin = (long long)split * p.keys_per_split;
  long long k_end = k_begin + p.keys_per_split;
  if (k_end > rs.n_cand) k_end = rs.n_cand;
  const uint32_t* keys = p.keys + (size_t)row * p.Tk;
  uint32_t gt = 0, eq = 0;
  for (long long i = k_begin + threadIdx.x; i < k_end; i += 256) {
    const uint32_t key = keys[i];
    gt += key > T;
    eq += key == T;
  }
  atomicAdd(&tot[0], gt);
  atomicAdd(&tot[1], eq);
  __syncthreads();
  if (threadIdx.x == 0) {
    cnt[0] = tot[0];
    cnt[1] = tot[1];
  }
}

// ---- 4. ordered compaction + window + padding ----------------------------------------------
__global__ __launch_bounds__(256) void tk_write_kernel(TopkDecodeParams p) {
  __shared__ uint32_t wsum[2][4];
  __shared__ long long base_sh[2];
  const int split = blockIdx.x, row = blockIdx.y;
  const RowSel rs = row_sel(p, row);
  int32_t* out = p.idx + (size_t)row * p.cap;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  if (split == p.n_split - 1) {
    // window positions after the k_eff selected candidates, then padding and the count
    const long long w0 = rs.t - p.window + 1 > 0 ? rs.t - p.window + 1 : 0;
    const int n_win = (int)(rs.t - w0 + 1);
    for (int i = threadIdx.x; i < p.cap - rs.k_eff; i += 256)
      out[rs.k_eff + i] = i < n_win ? (int32_t)(w0 + i) : -1;
    if (threadIdx.x == 0) p.cnt[row] = rs.k_eff + n_win;
  }
  if (rs.k_eff == 0) return;

  uint32_t T;
  int k_eq;
  threshold(p, row, rs.k_eff, &T, &k_eq);
  // offsets from the chunks before this one
  if (threadIdx.x == 0) {
    long long off = 0, eq_before = 0;
    const uint32_t* c = p.counts + (size_t)row * p.n_split * 2;
    for (int s = 0; s < split; s++) {
      const long long gt = c[2 * s], eq = c[2 * s + 1];
      long long take = k_eq - eq_before;
      take = take < 0 ? 0 : (take > eq ? eq : take);
      off += gt + take;
      eq_before += eq;
    }
    base_sh[0] = off;
    base_sh[1] = eq_before;
  }
  __syncthreads();
  long long off = base_sh[0], eq_seen = base_sh[1];
  const long long k_begin = (long long)split * p.keys_per_split;
  long long k_end = k_begin + p.keys_per_split;
  if (k_end > rs.n_cand) k_end = rs.n_cand;
  const uint32_t* keys = p.keys + (size_t)row * p.Tk;
  for (long long i0 = k_begin; i0 < k_end; i0 += 256) {
    const long long i = i0 + threadIdx.x;
    const uint32_t key = i < k_end ? keys[i] : 0u;
    const bool is_gt = i < k_end && key > T;
    const bool is_eq = i < k_end && key == T;
    // block-wide exclusive prefix of equal keys, in position order
    const unsigned long long beq = __ballot(is_eq);
    const unsigned long long lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const uint32_t eq_in_wave = __popcll(beq & lower);
    if (lane == 0) wsum[1][wave] = __popcll(beq);
    __syncthreads();
    uint32_t eq_prev = 0;
    for (int w = 0; w < wave; w++) eq_prev += wsum[1][w];
    const long long eq_rank = eq_seen + eq_prev + eq_in_wave;
    const bool take = is_gt || (is_eq && eq_rank < k_eq);
    const unsigned long long bt = __ballot(take);
    const uint32_t t_in_wave = __popcll(bt & lower);
    if (lane == 0) wsum[0][wave] = __popcll(bt);
    __syncthreads();
    uint32_t t_prev = 0, t_all = 0, eq_all = 0;
    for (int w = 0; w < 4; w++) {
      if (w < wave) t_prev += wsum[0][w];
      t_all += wsum[0][w];
      eq_all += wsum[1][w];
    }
    const long long slot = off + t_prev + t_in_wave;
    if (take && slot < rs.k_eff) out[slot] = (int32_t)i;
    off += t_all;
    eq_seen += eq_all;
    __syncthreads();
  }
}

template <int D, bool F32>
hipError_t launch_tk(const TopkDecodeParams& p, hipStream_t stream) {
  const size_t rows = (size_t)p.B * p.Tq * p.Hkv;
  const size_t hist_words = 3 * rows * kBins;
  zero_u32_kernel<<<(unsigned)((hist_words + 255) / 256 < 1024 ? (hist_words + 255) / 256 : 1024), 256, 0, stream>>>(p.hist, hist_words);
  tk_score_kernel<D, F32><<<dim3(p.n_split, p.B * p.Hkv * p.sets_per_bu), 256, 0, stream>>>(p);
  tk_pass_kernel<1><<<dim3(p.n_split, rows), 256, 0, stream>>>(p);
  tk_pass_kernel<2><<<dim3(p.n_split, rows), 256, 0, stream>>>(p);
  tk_count_kernel<<<dim3(p.n_split, rows), 256, 0, stream>>>(p);
  tk_write_kernel<<<dim3(p.n_split, rows), 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_decode(const TopkDecodeParams& p, int head_dim, bool in_f32,
                              hipStream_t stream) {
  if (head_dim == 128) return in_f32 ? launch_tk<128, true>(p, stream) : launch_tk<128, false>(p, stream);
  return in_f32 ? launch_tk<64, true>(p, stream) : launch_tk<64, false>(p, stream);
}

}  // namespace hs
