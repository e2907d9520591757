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
//   2. collect: the bin b1 holding the k-th key is found from the histogram; keys above b1 are
//      counted per chunk (all of them are taken), keys inside b1 go to a boundary list with
//      their positions;
//   3. finalize: radix passes over the boundary list's 64-bit values (key << 32 | ~position)
//      give the exact k1-th value V*, i.e. the key threshold T and the last position taken at
//      T (ties go to the lower position); per-chunk counts of taken keys follow;
//   4. write: ordered compaction per chunk (key > T, or key == T at a position <= the cut)
//      into the index list, which is therefore ascending; the window positions follow; -1
//      padding to the cap.
// Rows of at most 131072 keys run steps 2-4 in one workgroup per row instead (tk_select_kernel:
// the row's keys staged in LDS, two LDS radix levels below b1, then the same ordered
// compaction); only longer rows, whose few workgroups would leave the GPU idle, take 2-4 as
// separate kernels over key chunks.
// All steps are exact: nothing is dropped by an approximation.
#include "hs_device.h"
#include "hs_kernels.h"
#include "score_common.h"

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
  // KV head fastest, then split, then (batch, query chunk): see the row-attention kernel
  const int u = blockIdx.x % p.Hkv;
  const int split = (blockIdx.x / p.Hkv) % p.n_split;
  const int bq = blockIdx.x / (p.Hkv * p.n_split);
  const int sq = bq % p.sets_per_bu;
  const int b = bq / p.sets_per_bu;
  const int j0 = sq * p.q_per_set;
  const int nq = min(p.q_per_set, p.Tq - j0);
  const int nrows = nq * p.g;
  const int G = p.g / 4;  // lane groups per query

  for (int i = threadIdx.x; i < 4 * kBins; i += 256) (&hist[0][0])[i] = 0u;

  // A operand: Q rows (row r = jq * g + hh)
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

  // one 64-key tile already in registers
  auto score_tile = [&](const KTile<D, F32>& cur, long long tile) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const long long pos = tile + 16 * kb + rn;
      const f32x4 acc = score_block<D, F32>(cur, kb, qa, qf);
      // lane (key rn, group jg) holds rows 4jg..4jg+3 for key `pos`
      float v = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; e++) v = fmaxf(v, __builtin_fmaf(acc[e], p.scale_log2, -delta[e]));
      if (G >= 2) v = max_xor16(v);
      if (G >= 4) v = max_xor32(v);
      if (owner && pos <= last_cand && pos < k_end) {
        const uint32_t key = float_key(v);
        keys_row[pos] = key;
        atomicAdd(&hist[jq_own][key >> 21], 1u);
      }
    }
  };
  // Conditional prefetch: the compiler then waits for the prefetched tile before computing the
  // current one (no overlap inside a wave), which measured faster here than the peeled,
  // always-prefetching loop of the block score kernel (155 vs 162 us on the 7B decode step).
  KTile<D, F32> cur, nxt;
  long long tile = k_begin + 64LL * wave;
  if (tile < k_end) load_k_tile<D, F32>(cur, p.k, kv_base, kv_row_stride, tile, p.Tk, rn, jg);
  for (; tile < k_end; tile += 64LL * 4) {
    if (tile + 256 < k_end)
      load_k_tile<D, F32>(nxt, p.k, kv_base, kv_row_stride, tile + 256, p.Tk, rn, jg);
    score_tile(cur, tile);
    cur = nxt;
  }
  __syncthreads();
  for (int jq = 0; jq < nq; jq++) {
    uint32_t* gh = p.hist + ((size_t)(b * p.Tq + j0 + jq) * p.Hkv + u) * kBins;
    for (int i = threadIdx.x; i < kBins; i += 256) {
      const uint32_t c = hist[jq][i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

// ---- 1'. score from stored logits ---------------------------------------------------------
// Histogram increments of a wave, bin `bin` for the lanes with `take` (every lane of the wave
// active): the lanes that share the first taking lane's bin add with one atomic, the others
// one each.  A chunk's keys crowd into few bins, so most increments take the first path.
__device__ __forceinline__ void hist_add_wave(uint32_t* hist, uint32_t bin, bool take, int lane) {
  const unsigned long long act = __ballot(take);
  if (act == 0ull) return;
  const int first = __ffsll((long long)act) - 1;
  const uint32_t fb = __shfl(bin, first);
  const bool same = take && bin == fb;
  const unsigned long long m = __ballot(same);
  if (lane == first) atomicAdd(&hist[fb], (uint32_t)__popcll(m));
  if (take && !same) atomicAdd(&hist[bin], 1u);
}

// Same key as the score pass, from the raw dot products q.k that the full-attention pass stored
// ([B, Tq, Hq, Tk] fp32), so neither Q nor K is read again.  One workgroup per (row, key chunk).
// With 16-byte aligned rows (Tk a multiple of 4) and chunks of whole 1024-key passes, a thread
// takes 4 consecutive keys per pass and reads each head's 4 values with one 16-byte load (a
// wave reads 1 KB of a head row per load, a workgroup 4 KB), heads in groups of 16; otherwise a
// thread per key reads the G head values of its key (coalesced across the wave per head).
template <int G>
__global__ __launch_bounds__(256) void tk_logit_score_kernel(TopkDecodeParams p) {
  __shared__ uint32_t hist[kBins];
  __shared__ float dsh[64];
  const int split = blockIdx.x % p.n_split;
  const int row = blockIdx.x / p.n_split;  // (b * Tq + j) * Hkv + u
  const int u = row % p.Hkv;
  const int j = (row / p.Hkv) % p.Tq;
  const int b = row / (p.Hkv * p.Tq);
  for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = 0u;
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
  const long long t = p.q_off + j;
  const long long k_begin = (long long)split * p.keys_per_split;
  long long k_end = k_begin + p.keys_per_split;
  if (k_end > t - p.window + 1) k_end = t - p.window + 1;  // candidates 0 .. t - w
  const float* lg = p.logits + (((size_t)b * p.Tq + j) * p.Hq + (size_t)u * p.g) * p.Tk;
  uint32_t* keys_row = p.keys + (size_t)row * p.Tk;
  const bool vec = (p.Tk & 3) == 0 && (p.keys_per_split & 1023) == 0 &&
                   ((uintptr_t)p.logits & 15) == 0 && ((uintptr_t)p.keys & 15) == 0;
  if (vec) {
    constexpr int HC = G < 16 ? G : 16;  // heads per load group
    const int lane = threadIdx.x & 63;
    for (long long base = k_begin; base < k_end; base += 1024) {  // uniform trip count
      const long long pos = base + 4 * threadIdx.x;
      const bool in = pos < k_end;  // then pos + 3 < Tk (Tk and pos multiples of 4)
      float v[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c0 = 0; c0 < G; c0 += HC) {
        f32x4 x[HC];
#pragma unroll
        for (int i = 0; i < HC; i++)
          x[i] = (in && c0 + i < p.g) ? *(const f32x4*)(lg + (size_t)(c0 + i) * p.Tk + pos)
                                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < HC; i++)
#pragma unroll
          for (int e = 0; e < 4; e++)
            v[e] = fmaxf(v[e], __builtin_fmaf(x[i][e], p.scale_log2, -delta[c0 + i]));
      }
      uint32_t key[4];
#pragma unroll
      for (int e = 0; e < 4; e++) key[e] = float_key(v[e]);
      if (in) *(uint4*)(keys_row + pos) = make_uint4(key[0], key[1], key[2], key[3]);
#pragma unroll
      for (int e = 0; e < 4; e++) hist_add_wave(hist, key[e] >> 21, in && pos + e < k_end, lane);
    }
  } else {
  for (long long pos = k_begin + threadIdx.x; pos < k_end; pos += 256) {
    float x[G];
#pragma unroll
    for (int hh = 0; hh < G; hh++) x[hh] = hh < p.g ? lg[(size_t)hh * p.Tk + pos] : 0.f;
    float v = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < G; hh++) v = fmaxf(v, __builtin_fmaf(x[hh], p.scale_log2, -delta[hh]));
    const uint32_t key = float_key(v);
    keys_row[pos] = key;
    atomicAdd(&hist[key >> 21], 1u);
  }
  }
  __syncthreads();
  uint32_t* gh = p.hist + (size_t)row * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// ---- selection ----------------------------------------------------------------------------
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

// Scanning a 2048-bin histogram from the top bin down, find the bin that holds the k-th largest
// element and the rank (1-based) of that element inside the bin.  Wave 0 searches in two
// parallel steps: each lane sums a group of 32 bins and a scan over the lanes finds the group,
// then 32 lanes take one bin each of that group and a second scan finds the bin.  Every thread
// of the workgroup must call it (it synchronizes).  k is at least 1 and at most the total.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t x = __shfl_up(v, off, 64);
    if (lane >= off) v += x;
  }
  return v;
}

__device__ __forceinline__ void find_bin(const uint32_t* h, int k, int* bin_out, int* k_out) {
  __shared__ int res[2];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int top = kBins - 32 * lane;  // lane owns bins [top-32, top), lane 0 the highest
    uint32_t s = 0;
#pragma unroll
    for (int q = 1; q <= 32; q++) s += h[top - q];
    const uint32_t incl = wave_incl_scan(s, lane);
    const unsigned long long mg = __ballot(incl >= (uint32_t)k);
    const int gl = mg ? __ffsll((long long)mg) - 1 : 63;  // the group holding the k-th
    const uint32_t base = __shfl(incl - s, gl, 64);      // elements in higher groups
    const int gtop = kBins - 32 * gl;
    const uint32_t c = lane < 32 ? h[gtop - 1 - lane] : 0u;  // lane i: the group's i-th bin from the top
    const uint32_t ci = wave_incl_scan(c, lane);
    const unsigned long long mb = __ballot(lane < 32 && base + ci >= (uint32_t)k);
    const int bl = mb ? __ffsll((long long)mb) - 1 : 31;
    if (lane == bl) {
      res[0] = gtop - 1 - bl;
      res[1] = k - (int)(base + ci - c);
    }
  }
  __syncthreads();
  *bin_out = res[0];
  *k_out = res[1];
  __syncthreads();
}

// ---- 2. collect: per chunk, count keys above the boundary bin b1 (all taken) and append the
// keys inside it, with their positions, to the row's boundary list --------------------------
__global__ __launch_bounds__(256) void tk_collect_kernel(TopkDecodeParams p) {
  __shared__ uint32_t scan[256];
  __shared__ uint32_t base_sh, above_sh;
  __shared__ uint32_t hist[kBins];
  const int split = blockIdx.x, row = blockIdx.y;
  const RowSel rs = row_sel(p, row);
  if (rs.k_eff == 0) return;
  // the bin search reads the histogram bin by bin: from LDS, not over the memory latency
  for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = p.hist[(size_t)row * kBins + i];
  __syncthreads();
  int b1, k1;
  find_bin(hist, rs.k_eff, &b1, &k1);
  const long long k_begin = (long long)split * p.keys_per_sel;
  long long k_end = k_begin + p.keys_per_sel;
  if (k_end > rs.n_cand) k_end = rs.n_cand;
  const uint32_t* keys = p.keys + (size_t)row * p.Tk;
  // pass 1: per-thread counts of keys above b1 and inside b1 (8 loads in flight per trip)
  uint32_t above = 0, inside = 0;
  for (long long i0 = k_begin + threadIdx.x; i0 < k_end; i0 += 8 * 256) {
    uint32_t d[8];
#pragma unroll
    for (int r = 0; r < 8; r++) d[r] = i0 + 256 * r < k_end ? keys[i0 + 256 * r] >> 21 : 0u;
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const bool ok = i0 + 256 * r < k_end;
      above += ok && d[r] > (uint32_t)b1;
      inside += ok && d[r] == (uint32_t)b1;
    }
  }
  // exclusive scan of `inside` over the workgroup; one global reservation per workgroup
  scan[threadIdx.x] = inside;
  if (threadIdx.x == 0) above_sh = 0u;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t x = threadIdx.x >= off ? scan[threadIdx.x - off] : 0u;
    __syncthreads();
    scan[threadIdx.x] += x;
    __syncthreads();
  }
  atomicAdd(&above_sh, above);
  if (threadIdx.x == 255) base_sh = scan[255] ? atomicAdd(p.bcount + row, scan[255]) : 0u;
  __syncthreads();
  // pass 2: write this thread's boundary entries (key << 32 | ~position)
  unsigned long long* bl = p.blist + (size_t)row * p.Tk;
  uint32_t slot = base_sh + scan[threadIdx.x] - inside;
  for (long long i0 = k_begin + threadIdx.x; i0 < k_end && inside; i0 += 8 * 256) {
    uint32_t kv[8];
#pragma unroll
    for (int r = 0; r < 8; r++) kv[r] = i0 + 256 * r < k_end ? keys[i0 + 256 * r] : 0u;
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const long long i = i0 + 256 * r;
      if (i < k_end && (kv[r] >> 21) == (uint32_t)b1) {
        bl[slot++] = ((unsigned long long)kv[r] << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
        inside--;
      }
    }
  }
  if (threadIdx.x == 0) p.above[(size_t)row * p.sel_split + split] = above_sh;
}

// ---- 3. finalize: exact k1-th largest of the boundary list, by radix passes over the 64-bit
// value (key << 32 | ~position), so that ties in the key go to the lower position ------------
__global__ __launch_bounds__(256) void tk_finalize_kernel(TopkDecodeParams p) {
  constexpr int kStage = 4096;  // boundary entries staged in LDS when they fit
  __shared__ uint32_t hist[kBins];
  __shared__ unsigned long long stage[kStage];
  extern __shared__ uint32_t chunk_sel[];  // sel_split counters
  const int row = blockIdx.x;
  const RowSel rs = row_sel(p, row);
  if (rs.k_eff == 0) return;
  for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = p.hist[(size_t)row * kBins + i];
  __syncthreads();
  int b1, k1;
  find_bin(hist, rs.k_eff, &b1, &k1);  // ends with a barrier: hist is free again below
  const int m = (int)p.bcount[row];
  const unsigned long long* bl = p.blist + (size_t)row * p.Tk;
  if (m <= kStage) {
    for (int i = threadIdx.x; i < m; i += 256) stage[i] = bl[i];
    bl = stage;
  }
  // digits of V below the common 11-bit prefix: bits 52..42, 41..32, 31..21, 20..10, 9..0
  const int shifts[5] = {42, 32, 21, 10, 0};
  const int widths[5] = {11, 10, 11, 11, 10};
  unsigned long long prefix = (unsigned long long)b1 << 53, pmask = 0x7FFull << 53;
  int k = k1;
  for (int d = 0; d < 5; d++) {
    for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = 0u;
    __syncthreads();
    const unsigned long long dmask = (1ull << widths[d]) - 1ull;
    for (int i = threadIdx.x; i < m; i += 256) {
      const unsigned long long v = bl[i];
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shifts[d]) & dmask], 1u);
    }
    __syncthreads();
    int bin, kr;
    find_bin(hist, k, &bin, &kr);
    const bool all_taken = hist[bin] == (uint32_t)kr;
    prefix |= (unsigned long long)bin << shifts[d];
    pmask |= dmask << shifts[d];
    k = kr;
    // every entry with this prefix is taken: V >= prefix (lower bits 0) selects exactly them
    if (all_taken) break;
  }
  const unsigned long long vstar = prefix;
  for (int c = threadIdx.x; c < p.sel_split; c += 256) chunk_sel[c] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += 256) {
    const unsigned long long v = bl[i];
    if (v >= vstar) {
      const uint32_t pos = 0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull);
      atomicAdd(&chunk_sel[pos / p.keys_per_sel], 1u);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < p.sel_split; c += 256)
    p.counts[(size_t)row * p.sel_split + c] = p.above[(size_t)row * p.sel_split + c] + chunk_sel[c];
  if (threadIdx.x == 0) {
    // selection rule for every key: V >= V*, i.e. key > T, or key == T at position <= pos*
    p.state[2 * (size_t)row] = (uint32_t)(vstar >> 32);                              // T
    p.state[2 * (size_t)row + 1] = 0xFFFFFFFFu - (uint32_t)(vstar & 0xFFFFFFFFull);   // pos*
  }
}

// ---- 4. ordered compaction + window + padding ----------------------------------------------
__global__ __launch_bounds__(256) void tk_write_kernel(TopkDecodeParams p) {
  __shared__ uint32_t wsum[4];
  __shared__ long long base_sh;
  const int split = blockIdx.x, row = blockIdx.y;
  const RowSel rs = row_sel(p, row);
  int32_t* out = p.idx + (size_t)row * p.cap;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  if (split == p.sel_split - 1) {
    // window positions after the k_eff selected candidates, then padding and the count
    const long long w0 = rs.t - p.window + 1 > 0 ? rs.t - p.window + 1 : 0;
    const int n_win = (int)(rs.t - w0 + 1);
    for (int i = threadIdx.x; i < p.cap - rs.k_eff; i += 256)
      out[rs.k_eff + i] = i < n_win ? (int32_t)(w0 + i) : -1;
    if (threadIdx.x == 0) p.cnt[row] = rs.k_eff + n_win;
  }
  if (rs.k_eff == 0) return;
  const uint32_t T = p.state[2 * (size_t)row];
  const uint32_t pos_star = p.state[2 * (size_t)row + 1];
  if (threadIdx.x == 0) {
    long long off = 0;
    const uint32_t* c = p.counts + (size_t)row * p.sel_split;
    for (int s2 = 0; s2 < split; s2++) off += c[s2];
    base_sh = off;
  }
  __syncthreads();
  long long off = base_sh;
  const long long k_begin = (long long)split * p.keys_per_sel;
  long long k_end = k_begin + p.keys_per_sel;
  if (k_end > rs.n_cand) k_end = rs.n_cand;
  const uint32_t* keys = p.keys + (size_t)row * p.Tk;
  const unsigned long long lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (long long j0 = k_begin; j0 < k_end; j0 += 8 * 256) {
    uint32_t kv[8];  // the next 8 rounds' keys, loaded together
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const long long i = j0 + 256 * r + threadIdx.x;
      kv[r] = i < k_end ? keys[i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const long long i = j0 + 256 * r + threadIdx.x;
      const uint32_t key = kv[r];
      const bool take = i < k_end && (key > T || (key == T && (uint32_t)i <= pos_star));
      const unsigned long long bt = __ballot(take);
      if (lane == 0) wsum[wave] = __popcll(bt);
      __syncthreads();
      uint32_t t_prev = 0, t_all = 0;
      for (int w = 0; w < 4; w++) {
        if (w < wave) t_prev += wsum[w];
        t_all += wsum[w];
      }
      const long long slot = off + t_prev + __popcll(bt & lower);
      if (take && slot < rs.k_eff) out[slot] = (int32_t)i;
      off += t_all;
      __syncthreads();
    }
  }
}

// ---- 2-4 in one workgroup per row (rows of at most kSelMaxTiles tiles) --------------------
// The row's keys are staged in LDS, one tile of kSelTile keys at a time (longer rows reload the
// tile per pass).  Below the 11-bit bin b1 the remaining 21 key bits are resolved by two LDS
// histograms (bits 20..10, then 9..0), which give the exact key threshold T and the number k3
// of keys equal to T that are taken.  Keys equal to T are taken in position order, so the rule
// is the same as the chain's: key > T, or key == T among the first k3 such keys (ties go to
// the lower position).  Each lane owns 32 consecutive keys of the tile: a pass reads them in 8
// LDS loads and turns them into 32-bit masks (keys in the bin being refined; keys above T and
// equal to T), so that the per-key work (histogram atomics, ordered writes) runs over set bits
// only; slots come from mask popcounts plus one scan over the wave's lanes and one over the 16
// waves.  The kernel has few workgroups (one per row), so its instruction count per key sets
// its time.  Positions past the row's candidates are staged as key 0, which no finite score
// maps to (the smallest finite key is 0x00800000) and which lies below every bin refined.
constexpr int kSelThreads = 1024;
constexpr int kSelKeys = 32;                       // keys per lane
constexpr int kSelTile = kSelThreads * kSelKeys;   // 32768 keys
constexpr int kSelStride = kSelKeys + 4;           // LDS words per lane: 16-byte reads, no conflicts
constexpr uint32_t kAllTies = 0xFFFFFFFFu;         // every key equal to T is taken

__global__ __launch_bounds__(kSelThreads) void tk_select_kernel(TopkDecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t tile_keys[kSelThreads * kSelStride];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wsum[kSelThreads / 64];  // per wave: above | ties << 16
  const int row = blockIdx.x;
  const RowSel rs = row_sel(p, row);
  int32_t* out = p.idx + (size_t)row * p.cap;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    // window positions after the k_eff selected candidates, then padding and the count
    const long long w0 = rs.t - p.window + 1 > 0 ? rs.t - p.window + 1 : 0;
    const int n_win = (int)(rs.t - w0 + 1);
    for (int i = tid; i < p.cap - rs.k_eff; i += kSelThreads)
      out[rs.k_eff + i] = i < n_win ? (int32_t)(w0 + i) : -1;
    if (tid == 0) p.cnt[row] = rs.k_eff + n_win;
  }
  if (rs.k_eff == 0) return;
  const int n_cand = (int)rs.n_cand;
  const int n_tiles = (n_cand + kSelTile - 1) / kSelTile;
  // buffer descriptor over the row's keys, its range rounded up to whole 16-byte loads (the
  // at most 3 words past the row lie in the workspace): a load is wholly inside or returns 0
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.keys + (size_t)row * p.Tk), 0, ((n_cand + 3) & ~3) * 4, 0x00020000);
  // stage tile `tile`: thread t loads keys 4096 r + 4 t .. + 3 of the tile (coalesced) and
  // stores them as key i at word 36 (i / 32) + i % 32
  auto stage = [&](int tile) __attribute__((always_inline)) {
    u32x4 v[kSelKeys / 4];
#pragma unroll
    for (int r = 0; r < kSelKeys / 4; r++)
      v[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rsrc, (tile * kSelTile + 4096 * r + 4 * tid) * 4, 0, 0));
#pragma unroll
    for (int r = 0; r < kSelKeys / 4; r++) {
      const int i = 4096 * r + 4 * tid;
#pragma unroll
      for (int e = 0; e < 4; e++)
        if (tile * kSelTile + i + e >= n_cand) v[r][e] = 0u;
      *(u32x4*)(&tile_keys[(i >> 5) * kSelStride + (i & 31)]) = v[r];
    }
  };
  const uint32_t* my = tile_keys + tid * kSelStride;  // this lane's 32 consecutive keys
  auto mine = [&](uint32_t (&kk)[kSelKeys]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < kSelKeys / 4; m++) {
      const u32x4 v = *(const u32x4*)(my + 4 * m);
#pragma unroll
      for (int e = 0; e < 4; e++) kk[4 * m + e] = v[e];
    }
  };
  auto restage = [&](int tile) __attribute__((always_inline)) {
    if (n_tiles > 1) {
      __syncthreads();  // every lane is done with the previous tile
      stage(tile);
      __syncthreads();
    }
  };

  stage(0);
  // the row's top-11-bit histogram, scanned from LDS
  for (int i = tid; i < kBins; i += kSelThreads) hist[i] = p.hist[(size_t)row * kBins + i];
  __syncthreads();
  int b1, k1;
  find_bin(hist, rs.k_eff, &b1, &k1);
  uint32_t T = (uint32_t)b1 << 21, k3 = kAllTies;
  bool more = hist[b1] != (uint32_t)k1;
  // up to two radix levels: bits 20..10 under prefix b1, then bits 9..0 under prefix T >> 10
  int k = k1;
  for (int level = 0; level < 2 && more; level++) {
    const int shift = level == 0 ? 10 : 0, hi = level == 0 ? 21 : 10;
    const uint32_t prefix = T >> hi, mask = level == 0 ? 0x7FFu : 0x3FFu;
    __syncthreads();  // every thread is done with hist
    for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    for (int tile = 0; tile < n_tiles; tile++) {
      if (tile > 0 || level > 0) restage(tile);
      uint32_t kk[kSelKeys];
      mine(kk);
      uint32_t in_bin = 0;
#pragma unroll
      for (int j = 0; j < kSelKeys; j++) in_bin |= ((kk[j] >> hi) == prefix ? 1u : 0u) << j;
      while (in_bin) {
        const int j = __builtin_ctz(in_bin);
        in_bin &= in_bin - 1u;
        atomicAdd(&hist[(my[j] >> shift) & mask], 1u);
      }
    }
    __syncthreads();
    int bin, kb;
    find_bin(hist, k, &bin, &kb);
    T |= (uint32_t)bin << shift;
    if (level == 1) k3 = (uint32_t)kb;
    more = hist[bin] != (uint32_t)kb;
    k = kb;
  }

  // ordered compaction
  uint32_t carry_a = 0, carry_q = 0;  // keys above T and ties over earlier tiles
  const uint32_t k_eff = (uint32_t)rs.k_eff;  // bounds every slot, whatever the keys hold
  for (int tile = 0; tile < n_tiles; tile++) {
    restage(tile);
    uint32_t kk[kSelKeys];
    mine(kk);
    uint32_t ma = 0, mq = 0;  // this lane's keys above T, equal to T
#pragma unroll
    for (int j = 0; j < kSelKeys; j++) {
      ma |= (kk[j] > T ? 1u : 0u) << j;
      mq |= (kk[j] == T ? 1u : 0u) << j;
    }
    const uint32_t c = (uint32_t)__popc(ma) + ((uint32_t)__popc(mq) << 16);  // tile: < 2^16 each
    const uint32_t incl = wave_incl_scan(c, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = incl - c, total = 0;
    for (int w = 0; w < kSelThreads / 64; w++) {
      const uint32_t x = wsum[w];
      if (w < wave) before += x;
      total += x;
    }
    const uint32_t ia = carry_a + (before & 0xFFFFu), iq = carry_q + (before >> 16);
    carry_a += total & 0xFFFFu;
    carry_q += total >> 16;
    const int first = tile * kSelTile + kSelKeys * tid;
    uint32_t todo = ma | mq;
    while (todo) {
      const int j = __builtin_ctz(todo);
      todo &= todo - 1u;
      const uint32_t below = (1u << j) - 1u;
      const uint32_t qa = iq + (uint32_t)__popc(mq & below);  // ties before key j
      const uint32_t slot = ia + (uint32_t)__popc(ma & below) + (qa < k3 ? qa : k3);
      if ((((ma >> j) & 1u) || qa < k3) && slot < k_eff) out[slot] = first + j;
    }
    __syncthreads();  // wsum is rewritten by the next tile
  }
}

// Steps 2-4: one workgroup per row while a row spans at most kSelMaxTiles tiles (each
// workgroup then reads its keys at most three times); longer rows, whose few workgroups would
// leave most of the GPU idle, take the chain of collect / finalize / write over key chunks.
constexpr int kSelMaxTiles = 4;

void launch_select(const TopkDecodeParams& p, size_t rows, hipStream_t stream) {
  if (!topk_decode_uses_chain(p.Tk)) {
    tk_select_kernel<<<dim3((unsigned)rows), kSelThreads, 0, stream>>>(p);
    return;
  }
  tk_collect_kernel<<<dim3(p.sel_split, rows), 256, 0, stream>>>(p);
  tk_finalize_kernel<<<dim3((unsigned)rows), 256, p.sel_split * sizeof(uint32_t), stream>>>(p);
  tk_write_kernel<<<dim3(p.sel_split, rows), 256, 0, stream>>>(p);
}

template <int D, bool F32>
hipError_t launch_tk(const TopkDecodeParams& p, hipStream_t stream) {
  const size_t rows = (size_t)p.B * p.Tq * p.Hkv;
  const size_t zero_words = rows * kBins + rows;  // first histograms, then boundary counters
  zero_u32_kernel<<<(unsigned)((zero_words + 255) / 256 < 1024 ? (zero_words + 255) / 256 : 1024), 256, 0, stream>>>(p.hist, zero_words);
  tk_score_kernel<D, F32><<<dim3(p.n_split * p.B * p.Hkv * p.sets_per_bu), 256, 0, stream>>>(p);
  launch_select(p, rows, stream);
  return hipGetLastError();
}

template <int G>
hipError_t launch_tk_logits(const TopkDecodeParams& p, hipStream_t stream) {
  const size_t rows = (size_t)p.B * p.Tq * p.Hkv;
  const size_t zero_words = rows * kBins + rows;
  zero_u32_kernel<<<(unsigned)((zero_words + 255) / 256 < 1024 ? (zero_words + 255) / 256 : 1024), 256, 0, stream>>>(p.hist, zero_words);
  tk_logit_score_kernel<G><<<dim3((unsigned)(p.n_split * rows)), 256, 0, stream>>>(p);
  launch_select(p, rows, stream);
  return hipGetLastError();
}

}  // namespace

bool topk_decode_uses_chain(long long Tk) { return Tk > (long long)kSelMaxTiles * kSelTile; }

hipError_t launch_topk_from_logits(const TopkDecodeParams& p, hipStream_t stream) {
  switch (p.g) {
    case 1: return launch_tk_logits<1>(p, stream);
    case 2: return launch_tk_logits<2>(p, stream);
    case 3: return launch_tk_logits<3>(p, stream);
    case 4: return launch_tk_logits<4>(p, stream);
    case 5: return launch_tk_logits<5>(p, stream);
    case 6: return launch_tk_logits<6>(p, stream);
    case 7: return launch_tk_logits<7>(p, stream);
    case 8: return launch_tk_logits<8>(p, stream);
    case 9: return launch_tk_logits<9>(p, stream);
    case 10: return launch_tk_logits<10>(p, stream);
    case 11: return launch_tk_logits<11>(p, stream);
    case 12: return launch_tk_logits<12>(p, stream);
    case 13: return launch_tk_logits<13>(p, stream);
    case 14: return launch_tk_logits<14>(p, stream);
    case 15: return launch_tk_logits<15>(p, stream);
    case 16: return launch_tk_logits<16>(p, stream);
    case 32: return launch_tk_logits<32>(p, stream);
    case 48: return launch_tk_logits<48>(p, stream);
    case 64: return launch_tk_logits<64>(p, stream);
  }
  // other group sizes run on the next larger instantiation, the extra heads masked
  if (p.g < 32) return launch_tk_logits<32>(p, stream);
  if (p.g < 48) return launch_tk_logits<48>(p, stream);
  if (p.g < 64) return launch_tk_logits<64>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_topk_decode(const TopkDecodeParams& p, int head_dim, bool in_f32,
                              hipStream_t stream) {
  if (head_dim == 128) return in_f32 ? launch_tk<128, true>(p, stream) : launch_tk<128, false>(p, stream);
  return in_f32 ? launch_tk<64, true>(p, stream) : launch_tk<64, false>(p, stream);
}

}  // namespace hs
