// topk_prefill.hip -- exact token and block selection for many queries per KV head (prefill),
// without storing any per-key score: scores are recomputed tile by tile and selected on the fly.
//
// Scores [P2 "Extracting block scores from exact attention"; P2 "GQA: the group shares one index
// set"; P4 section 3.2]:
//   token  s_i = max_{h in group} exp(a^h_i - LSE^h)            (HySparse2, P1 section 4.2; P5)
//   block  S_r = max over the block's keys i <= t of s_i        (HySparse, P2 TopK equation)
// ranked in the log2 domain as max_h(a^h * tau * log2 e - (LSE^h * log2 e - C)) with a per-query
// integer C, exactly as in the decode kernels, and compared as 64-bit values
// V = (order-preserving score bits << 32) | ~position (or ~block id): equal scores prefer the
// lower position.
//
// Tiling: a workgroup owns 256 (query, head) rows of one KV head (256/g queries, all g heads),
// 4 waves of 64 rows; 64-key K tiles are double-buffered in LDS and shared by all rows.
// S = Q K^T on MFMA (A = Q rows resident, B = K^T from LDS).  Rows are packed so that a lane
// holds, for one key, four heads of one query in each of the g/4 MFMA blocks of that query:
// the group maximum over the heads is taken inside the lane, with no cross-lane traffic.
//
// Token mode: each query keeps a candidate buffer (2048 entries) in the workspace.  A key enters
// it if it is a candidate (position <= t - w) and V >= theta, the query's running threshold.
// When the buffer is nearly full, the query's wave compacts it exactly: a radix select (8-bit
// digits; entries in registers, histogram in LDS) finds the k-th largest V, theta becomes that
// value (or the lower bound of a bin taken whole), and only entries >= theta stay.  Every key
// dropped is below k kept keys, so the final top-k is exact.  At the end the k positions are
// sorted (bitonic, in LDS) and the forced window is appended.
// Block mode (blocks of 16, 32 or 64 keys): each query keeps its best n blocks in registers,
// spread over the 16 lanes that hold its keys; at each block boundary the block's V replaces
// the list minimum (found with four lane exchanges) when it is larger.
#include "hs_device.h"
#include "hs_kernels.h"

namespace hs {
namespace {

constexpr int kThreads = 256;  // 4 waves of 64 rows
constexpr int kRowsWG = 256;
constexpr int kBN = 64;
constexpr int kBufCap = 2048;          // token candidates per query
constexpr int kNPL = kBufCap / 64;     // buffer entries per lane during a compaction
// Entries a compaction before the end may keep beyond k (the rest of the k-th entry's bin);
// k + slack must leave room for a tile's appends (at most 64 per query).
constexpr int kCompactSlack = 256;
constexpr int kSortCap = 1024;         // largest k_global of the token mode
constexpr int kMaxBlocks = 64;         // largest n_blocks

template <int D, bool F32>
struct PsCfg {
  static constexpr int Elem = F32 ? 4 : 2;
  static constexpr int KStr = F32 ? D + 4 : D + 8;  // K tile row stride (elements)
  static constexpr int KK = F32 ? D / 4 : D / 32;   // MFMA steps over d
  static constexpr int CPR = D * Elem / 16;         // 16-byte chunks per row
  static constexpr int LPT = kBN * CPR / kThreads;  // chunks per thread per tile
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Loads of data this kernel wrote earlier (candidate buffers): agent-scope atomic loads do not
// return stale copies from the per-CU cache.  Callers first complete their own stores with a
// workgroup-scope release fence.
__device__ __forceinline__ unsigned long long ld_coherent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide: scanning 256 LDS bins from the top, the bin holding the k-th largest element, the
// rank of that element inside the bin, and the bin's count.
__device__ __forceinline__ void wave_find_bin(const uint32_t* h, int k, int lane, int* bin,
                                              int* kr, uint32_t* bin_count) {
  uint32_t c[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    c[q] = h[255 - 4 * lane - q];  // lane 0 owns the highest bins
    s += c[q];
  }
  uint32_t incl = s;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t x = __shfl_up(incl, off, 64);
    if (lane >= off) incl += x;
  }
  const uint32_t excl = incl - s;
  int my_bin = -1, my_kr = 0;
  uint32_t my_cnt = 0;
  if ((long long)excl < k && (long long)k <= (long long)incl) {
    uint32_t cum = excl;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      if (my_bin < 0 && (long long)cum + c[q] >= k) {
        my_bin = 255 - 4 * lane - q;
        my_kr = k - (int)cum;
        my_cnt = c[q];
      }
      cum += c[q];
    }
  }
  const unsigned long long who = __ballot(my_bin >= 0);
  const int src = who ? (__ffsll((long long)who) - 1) : 0;
  *bin = __shfl(my_bin, src, 64);
  *kr = __shfl(my_kr, src, 64);
  *bin_count = __shfl(my_cnt, src, 64);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Keep exactly the k largest of the n (> k) entries of `buf`; returns the new threshold theta
// (entries >= theta are the ones kept, compacted to buf[0..k)).  Wave-wide.  If `sorted_pos`
// is given, the kept positions (~low word) are also written there, unordered.
__device__ unsigned long long wave_compact(unsigned long long* buf, int n, int k, int lane,
                                           uint32_t* hist, int* kept_pos, int slack,
                                           int* kept_out) {
  unsigned long long v[kNPL];
#pragma unroll
  for (int i = 0; i < kNPL; i++) {
    const int idx = lane + 64 * i;
    v[i] = idx < n ? ld_coherent(buf + idx) : 0ull;
  }
  // Start below the bits that all entries share: the entries are scores near the top of the
  // row, so their leading bits coincide, and a histogram of them would send every lane's atomic
  // to the same LDS bin.
  unsigned long long vmin = ~0ull, vmax = 0ull;
#pragma unroll
  for (int i = 0; i < kNPL; i++) {
    if (v[i] != 0ull) {
      vmin = v[i] < vmin ? v[i] : vmin;
      vmax = v[i] > vmax ? v[i] : vmax;
    }
  }
  for (int m = 1; m < 64; m <<= 1) {
    const unsigned long long a = shfl_xor_u64(vmin, m), c = shfl_xor_u64(vmax, m);
    vmin = a < vmin ? a : vmin;
    vmax = c > vmax ? c : vmax;
  }
  int start = 56;  // first 8-bit digit that holds a differing bit
  if (vmin < vmax) start = ((63 - __clzll((long long)(vmin ^ vmax))) / 8) * 8;
  unsigned long long pmask = start == 56 ? 0ull : ~((1ull << (start + 8)) - 1ull);
  unsigned long long prefix = vmin & pmask;
  int kk = k;
  for (int shift = start; shift >= 0; shift -= 8) {
#pragma unroll
    for (int q = 0; q < 4; q++) hist[4 * lane + q] = 0u;
    wave_sync_lds();
#pragma unroll
    for (int i = 0; i < kNPL; i++)
      if (v[i] != 0ull && (v[i] & pmask) == prefix) atomicAdd(&hist[(v[i] >> shift) & 255ull], 1u);
    wave_sync_lds();
    int bin, kr;
    uint32_t cnt;
    wave_find_bin(hist, kk, lane, &bin, &kr, &cnt);
    prefix |= (unsigned long long)bin << shift;
    pmask |= 255ull << shift;
    kk = kr;
    wave_sync_lds();
    if (cnt == (uint32_t)kr) break;  // the bin is taken whole: V >= prefix selects exactly k
    // A running threshold only has to stay at or below the k-th value: keeping the whole bin
    // of the k-th entry (at most `slack` entries beyond k) ends the select after one pass.
    if (slack > 0 && (int)cnt - kr <= slack) break;
  }
  const unsigned long long theta = prefix;
  int base = 0;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < kNPL; i++) {
    const bool keep = v[i] != 0ull && v[i] >= theta;
    const unsigned long long bm = __ballot(keep);
    const int slot = base + __popcll(bm & below);
    if (keep) {
      buf[slot] = v[i];
      if (kept_pos) kept_pos[slot] = (int)(0xFFFFFFFFu - (uint32_t)(v[i] & 0xFFFFFFFFull));
    }
    base += __popcll(bm);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // stores complete before reloads
  *kept_out = base;
  return theta;
}

// Ascending bitonic sort of M (a power of two) ints in this wave's LDS area.
__device__ void wave_bitonic_sort(int* a, int M, int lane) {
  for (int kk = 2; kk <= M; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = lane; i < M; i += 64) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const int x = a[i], y = a[ixj];
          const bool up = (i & kk) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      wave_sync_lds();
    }
  }
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// G: query heads per KV head (4, 8 or 16).  NE: block-list entries per lane (n_blocks <= 16 NE).
template <int D, bool F32, bool BLOCK, int G, int NE>
__global__ __launch_bounds__(kThreads, F32 ? 1 : 2) void pf_select_kernel(PrefillSelectParams p) {
  using C = PsCfg<D, F32>;
  constexpr int NW = kThreads / 64;  // waves
  constexpr int HQ = G / 4;          // head quarters per query
  constexpr int QG = 4 / HQ;         // query groups per wave
  constexpr int QW = 4 * QG;         // queries per wave (64 / G)
  constexpr int QPW = NW * QW;       // queries per workgroup (256 / G)
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][kBN * C::KStr * C::Elem];
  __shared__ uint32_t whist[BLOCK ? 1 : NW][256];
  __shared__ unsigned long long blist[BLOCK ? NW * QW : 1][BLOCK ? 16 * NE : 1];
  __shared__ int sortbuf[BLOCK ? 1 : NW][BLOCK ? 1 : kSortCap];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rn = lane & 15, jg = lane >> 4;
  // Row packing, head-quarter major: the wave's 64 rows are 4 MFMA blocks; block rb holds heads
  // 4hq..4hq+3 of the 4 queries of query group qg (rb = qg * HQ + hq), MFMA row 4j+e being
  // query 4qg+j, head 4hq+e.  The S = Q K^T output then gives lane (key, j) heads 4hq..4hq+3 of
  // query 4qg+j in every block of the group: the group maximum over all G heads is in-lane.
  const int n_qt = (p.Tq + QPW - 1) / QPW;
  const int u = blockIdx.x % p.Hkv;
  const int qt = n_qt - 1 - (int)((blockIdx.x / p.Hkv) % n_qt);
  const int b = blockIdx.x / (p.Hkv * n_qt);
  const int j0 = qt * QPW;
  const int nq = min(QPW, p.Tq - j0);
  const int tq0 = (int)p.q_off + j0;  // positions fit in 31 bits
  const int t_max = tq0 + nq - 1;
  const int wq0 = wave * QW;  // first workgroup query of this wave

  constexpr int KK = C::KK;
  bf16x8 qa[4][F32 ? 1 : KK];
  float qf[4][F32 ? KK : 1];
  // A operand: lane row rn = 4j + e of block rb -> query 4qg + j, head 4hq + e.  Reloaded after
  // buffer compactions, which then need no registers of their own for it.
  auto load_q = [&]() {
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      const int qg = rb / HQ, hq = rb % HQ;
      const int jq = wq0 + 4 * qg + rn / 4;
      const int hh = 4 * hq + rn % 4;
      const bool ok = jq < nq;
      const size_t qoff = (((size_t)b * p.Tq + j0 + (ok ? jq : 0)) * p.Hq + u * G + hh) * D;
      if constexpr (!F32) {
        const uint16_t* qp = (const uint16_t*)p.q + qoff;
#pragma unroll
        for (int kk = 0; kk < KK; kk++) {
          u32x4 raw = ok ? *(const u32x4*)(qp + 32 * kk + 8 * jg) : u32x4{0, 0, 0, 0};
          qa[rb][kk] = __builtin_bit_cast(bf16x8, raw);
        }
      } else {
        const float* qp = (const float*)p.q + qoff + jg * KK;
#pragma unroll
        for (int s2 = 0; s2 < KK; s2++) qf[rb][s2] = ok ? qp[s2] : 0.f;
      }
    }
  };
  load_q();
  float delta[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++) {
    const int qg = rb / HQ, hq = rb % HQ;
    {  // output rows of lane group jg: query 4qg + jg, heads 4hq + e
      const int jq = wq0 + 4 * qg + jg;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        if (jq < nq) {
          const int j = j0 + jq, hh = 4 * hq + e;
          const double l2 = (double)p.lse[((size_t)b * p.Hq + u * G + hh) * p.Tq + j] * 1.4426950408889634;
          const double Cq = rint((double)p.lse[((size_t)b * p.Hq + u * G) * p.Tq + j] * 1.4426950408889634);
          delta[rb][e] = (float)(l2 - Cq);
        } else {
          delta[rb][e] = INFINITY;  // queries past the last one never score
        }
      }
    }
  }
  // this lane's query in each query group
  int t_q[QG];
  bool q_ok[QG];
#pragma unroll
  for (int qg = 0; qg < QG; qg++) {
    const int jq = wq0 + 4 * qg + jg;
    q_ok[qg] = jq < nq;
    t_q[qg] = tq0 + jq;
  }

  // token mode: buffer fill and threshold of this lane's queries (the same in its 16 lanes)
  int cnt[QG];
  unsigned long long th[QG];
  float thf[QG];
  // block mode: running block maxima and the best-n list, slot e*16 + rn in L[qg][e]; an empty
  // slot holds its own index (below every real entry, so empties fill in slot order), slots past
  // n_blocks hold ~0 and are never replaced.
  float bmax[QG];
  unsigned long long L[QG][NE];
#pragma unroll
  for (int qg = 0; qg < QG; qg++) {
    cnt[qg] = 0;
    th[qg] = 0ull;
    thf[qg] = -INFINITY;
    bmax[qg] = -INFINITY;
#pragma unroll
    for (int e = 0; e < NE; e++) {
      const int slot = 16 * e + rn;
      L[qg][e] = slot < p.n_blocks ? (unsigned long long)slot : ~0ull;
    }
  }
  const int bshift = BLOCK ? __ffs(p.block) - 1 : 0;  // blocks of 16, 32 or 64 keys

  const size_t kv_row_stride = (size_t)p.Hkv * D;
  const unsigned char* kbase =
      (const unsigned char*)p.k + ((size_t)b * p.Tk * p.Hkv + u) * D * C::Elem;
  const int key_last = BLOCK ? t_max : t_max - p.window;  // last key any query needs
  const int n_tiles = key_last < 0 ? 0 : key_last / kBN + 1;
  u32x4 kreg[C::LPT];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::LPT; i++) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / C::CPR, ch = c % C::CPR;
      const int key = min(t * kBN + row, key_last);
      kreg[i] = *(const u32x4*)(kbase + ((size_t)key * kv_row_stride) * C::Elem + ch * 16);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LPT; i++) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / C::CPR, ch = c % C::CPR;
      *(u32x4*)(&ktile[buf][(row * C::KStr) * C::Elem + ch * 16]) = kreg[i];
    }
  };
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const unsigned long long qmask = 0xFFFFull << (16 * jg);  // lanes of this lane's query
  auto buf_of = [&](int wq) {
    return p.tbuf + ((size_t)((size_t)b * p.Tq + j0 + wq0 + wq) * p.Hkv + u) * kBufCap;
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  // Complete every load issued so far (the resident Q operand among them) here: otherwise the
  // first use of Q inside the loop leaves a wait for all loads in every iteration, and the next
  // K tile's loads would never overlap the current tile's work.
  __builtin_amdgcn_s_waitcnt(0);
  for (int t = 0; t < n_tiles; t++) {
    const int buf = t & 1;
    const int key0 = t * kBN;

    if constexpr (!BLOCK) {  // before the next tile's loads: their registers are free here
      // make room: compact every nearly full buffer of this wave's queries
      bool full = false;
#pragma unroll
      for (int qg = 0; qg < QG; qg++) full |= cnt[qg] > kBufCap - kBN;
      if (__ballot(full)) {
#pragma unroll
        for (int qg = 0; qg < QG; qg++) {
          for (int jj = 0; jj < 4; jj++) {
            const int n = __shfl(cnt[qg], 16 * jj, 64);
            if (n > kBufCap - kBN) {
              int kept;
              const unsigned long long tnew = wave_compact(buf_of(4 * qg + jj), n, p.k_global,
                                                           lane, whist[wave], nullptr,
                                                           kCompactSlack, &kept);
              if (jg == jj) {
                cnt[qg] = kept;
                th[qg] = tnew;
                const uint32_t hi = (uint32_t)(tnew >> 32);
                thf[qg] = hi ? key_to_float(hi) : -INFINITY;
              }
            }
          }
        }
        load_q();
        __builtin_amdgcn_s_waitcnt(0);
      }
    }
    if (t + 1 < n_tiles) load_tile(t + 1);

#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      f32x4 acc[4];
#pragma unroll
      for (int rb = 0; rb < 4; rb++) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!F32) {
        const uint16_t* kt = (const uint16_t*)ktile[buf];
#pragma unroll
        for (int kk = 0; kk < KK; kk++) {
          const bf16x8 kbv = *(const bf16x8*)(kt + (16 * kb + rn) * C::KStr + 32 * kk + 8 * jg);
#pragma unroll
          for (int rb = 0; rb < 4; rb++) acc[rb] = mfma_bf16(qa[rb][kk], kbv, acc[rb]);
        }
      } else {
        const float* kt = (const float*)ktile[buf];
#pragma unroll
        for (int s2 = 0; s2 < KK; s2++) {
          const float kv = kt[(16 * kb + rn) * C::KStr + jg * KK + s2];
#pragma unroll
          for (int rb = 0; rb < 4; rb++) acc[rb] = mfma_f32(qf[rb][s2], kv, acc[rb]);
        }
      }
      const int g0 = key0 + 16 * kb;
      const int pos = g0 + rn;
#pragma unroll
      for (int qg = 0; qg < QG; qg++) {
        float v = -INFINITY;
#pragma unroll
        for (int hq = 0; hq < HQ; hq++) {
          const int rb = qg * HQ + hq;
#pragma unroll
          for (int e = 0; e < 4; e++) v = fmaxf(v, __builtin_fmaf(acc[rb][e], p.scale_log2, -delta[rb][e]));
        }
        if constexpr (!BLOCK) {
          bool take = false;
          if (q_ok[qg] && pos <= t_q[qg] - p.window && v >= thf[qg]) {
            if (v > thf[qg]) {
              take = true;
            } else {  // equal to the float filter: decide on the exact 64-bit value
              const unsigned long long V = ((unsigned long long)float_key(v) << 32) |
                                           (unsigned long long)(0xFFFFFFFFu - (uint32_t)pos);
              take = V >= th[qg];
            }
          }
          const unsigned long long bm = __ballot(take);
          if (bm) {
            if (take) {
              const int slot = cnt[qg] + __popcll(bm & qmask & below);
              buf_of(4 * qg + jg)[slot] = ((unsigned long long)float_key(v) << 32) |
                                          (unsigned long long)(0xFFFFFFFFu - (uint32_t)pos);
            }
            cnt[qg] += __popcll(bm & qmask);
          }
        } else {
          // running maximum of the current block (keys past the query are masked)
          bmax[qg] = fmaxf(bmax[qg], (q_ok[qg] && pos <= t_q[qg]) ? v : -INFINITY);
          if (((g0 + 16) & (p.block - 1)) == 0) {  // block boundary: the same for every lane
            const float bv = max16(bmax[qg]);
            const int bstart = g0 + 16 - p.block;
            const unsigned long long V = ((unsigned long long)float_key(bv) << 32) |
                                         (unsigned long long)(0xFFFFFFFFu - (uint32_t)(bstart >> bshift));
            // minimum of the query's list (16 lanes x NE entries, all distinct)
            unsigned long long mn = L[qg][0];
#pragma unroll
            for (int e = 1; e < NE; e++) mn = L[qg][e] < mn ? L[qg][e] : mn;
            const unsigned long long gmn = min16_u64(mn);
            if (q_ok[qg] && bstart <= t_q[qg] && V > gmn && mn == gmn) {
#pragma unroll
              for (int e = 0; e < NE; e++)
                if (L[qg][e] == gmn) L[qg][e] = V;
            }
            bmax[qg] = -INFINITY;
          }
        }
      }
    }
    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- outputs, one query at a time per wave ----
  if constexpr (BLOCK) {
#pragma unroll
    for (int qg = 0; qg < QG; qg++)
#pragma unroll
      for (int e = 0; e < NE; e++) blist[wave * QW + 4 * qg + jg][16 * e + rn] = L[qg][e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int qg = 0; qg < QG; qg++) {
    for (int jj = 0; jj < 4; jj++) {
      const int wq = 4 * qg + jj;
      const int jq = wq0 + wq;
      if (jq >= nq) break;
      const int t = tq0 + jq;
      const long long row = ((long long)b * p.Tq + j0 + jq) * p.Hkv + u;
      if constexpr (!BLOCK) {
        const int n_cand = max(t - p.window + 1, 0);
        const int k_eff = min(n_cand, p.k_global);
        unsigned long long* bufq = buf_of(wq);
        int* sb = sortbuf[wave];
        const int n = __shfl(cnt[qg], 16 * jj, 64);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // appends complete before reloads
        if (n > k_eff) {
          int kept_final;
          wave_compact(bufq, n, k_eff, lane, whist[wave], sb, 0, &kept_final);
        } else {
          for (int i = lane; i < n; i += 64)
            sb[i] = (int)(0xFFFFFFFFu - (uint32_t)(ld_coherent(bufq + i) & 0xFFFFFFFFull));
        }
        int M = 1;
        while (M < k_eff) M <<= 1;
        for (int i = k_eff + lane; i < M; i += 64) sb[i] = 0x7FFFFFFF;
        wave_sync_lds();
        wave_bitonic_sort(sb, M, lane);
        int32_t* out = p.idx + (size_t)row * p.cap;
        const int w0 = max(t - p.window + 1, 0);
        const int n_win = t - w0 + 1;
        for (int i = lane; i < p.cap; i += 64) {
          int32_t val = -1;
          if (i < k_eff) val = sb[i];
          else if (i < k_eff + n_win) val = w0 + (i - k_eff);
          out[i] = val;
        }
        if (lane == 0) p.cnt[row] = k_eff + n_win;
        wave_sync_lds();
      } else {
        const int n_take = min((t >> bshift) + 1, p.n_blocks);
        const unsigned long long* Lq = blist[wave * QW + wq];
        int32_t* out = p.idx + (size_t)row * p.n_blocks;
        // real entries occupy slots 0 .. n_take-1 (empties are replaced in slot order)
        if (lane < p.n_blocks) {
          if (lane < n_take) {
            const int id = (int)(0xFFFFFFFFu - (uint32_t)(Lq[lane] & 0xFFFFFFFFull));
            int rank = 0;
            for (int o = 0; o < n_take; o++)
              rank += (int)(0xFFFFFFFFu - (uint32_t)(Lq[o] & 0xFFFFFFFFull)) < id;
            out[rank] = id;
          } else {
            out[lane] = -1;
          }
        }
        if (lane == 0) p.cnt[row] = n_take;
      }
    }
  }
}

template <int D, bool F32, bool BLOCK, int G>
void launch_g(const PrefillSelectParams& p, dim3 grid, hipStream_t stream) {
  if constexpr (BLOCK) {
    if (p.n_blocks > 16) {
      pf_select_kernel<D, F32, BLOCK, G, 4><<<grid, kThreads, 0, stream>>>(p);
      return;
    }
  }
  pf_select_kernel<D, F32, BLOCK, G, 1><<<grid, kThreads, 0, stream>>>(p);
}

template <int D, bool F32, bool BLOCK>
void launch_dfb(const PrefillSelectParams& p, hipStream_t stream) {
  const int qpw = kRowsWG / p.g;  // queries per workgroup
  const int n_qt = (p.Tq + qpw - 1) / qpw;
  const dim3 grid(p.B * p.Hkv * n_qt);
  if (p.g == 4)
    launch_g<D, F32, BLOCK, 4>(p, grid, stream);
  else if (p.g == 8)
    launch_g<D, F32, BLOCK, 8>(p, grid, stream);
  else
    launch_g<D, F32, BLOCK, 16>(p, grid, stream);
}

}  // namespace

int prefill_select_buffer_cap() { return kBufCap; }
int prefill_select_max_k() { return kSortCap; }

hipError_t launch_prefill_select(const PrefillSelectParams& p, int head_dim, bool in_f32,
                                 bool block_mode, hipStream_t stream) {
  if (p.g != 4 && p.g != 8 && p.g != 16) return hipErrorInvalidValue;
  if (block_mode && (p.block < 16 || p.block > 64 || (p.block & (p.block - 1)) ||
                     p.n_blocks < 1 || p.n_blocks > kMaxBlocks))
    return hipErrorInvalidValue;
  if (head_dim == 128) {
    if (in_f32) {
      if (block_mode) launch_dfb<128, true, true>(p, stream); else launch_dfb<128, true, false>(p, stream);
    } else {
      if (block_mode) launch_dfb<128, false, true>(p, stream); else launch_dfb<128, false, false>(p, stream);
    }
  } else {
    if (in_f32) {
      if (block_mode) launch_dfb<64, true, true>(p, stream); else launch_dfb<64, true, false>(p, stream);
    } else {
      if (block_mode) launch_dfb<64, false, true>(p, stream); else launch_dfb<64, false, false>(p, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace hs
