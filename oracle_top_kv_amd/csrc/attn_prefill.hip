// attn_prefill.hip -- full causal GQA attention for many queries per KV head (prefill):
// O and LSE [P2 "Extracting block scores from exact attention", attention equations;
// P4 section 3.2, the tiled loop of Algorithm 1 without its score output].
//
// A workgroup owns 256 (query, head) rows of one KV head: 256/g consecutive queries times the
// g heads of the group, so every K/V tile staged in LDS serves all heads of the group (256 rows
// per 64-key tile: 128 flop per byte of K/V moved from L2).  Each of the 8 waves owns 32 rows,
// one column block of v_mfma_f32_32x32x16_bf16.  Per 64-key tile:
//   S^T = K Q^T   A = K (32 keys x 16 d) from LDS, B = Q^T resident in registers; lane l then
//                 holds row l%32 for 32 of the tile's keys, the other 32 sit in lane l^32
//   online softmax in the log2 domain (scale folded into the exponent's FMA); the row maximum is
//                 an in-lane max3 chain plus one v_permlane32_swap
//   O^T += V^T P^T  B = P^T straight from the S^T accumulator (bf16), A = V^T from the
//                 row-major LDS tile with ds_read_b64_tr_b16 (keys in the accumulator's order)
// K/V tiles are double-buffered: the next tile's rows are loaded into registers while the
// current tile is computed, then stored to the other buffer; one barrier per tile.  Only tiles
// that reach past the earliest query position of the workgroup apply the causal mask.
//
// BSEL: the HySparse block selection in the same pass, for blocks of 64 keys (one tile).  The
// pages compute the block scores inside the attention loop from each tile's row maximum and
// normalize them once the LSE is known [P4 Algorithm 1; P2 "Extracting block scores from exact
// attention" and "Why normalize scores for TopK"].  Here no score matrix is stored: within one
// head, p = exp(a - LSE) ranks like the raw logit a, so each row keeps its own best n blocks by
// raw tile maximum as the tiles stream past (an exact running top-n); at the end the g rows of a
// query merge their lists with the normalized scores.  The merge is exact: a block among the
// group's best n is among the best n of the head that attains its group maximum.
#include <type_traits>

#include "hs_device.h"
#include "hs_kernels.h"

namespace hs {
namespace {

constexpr int kThreads = 512;  // 8 waves (head sizes up to 128; the block-selection merge)
constexpr int kBN = 64;  // keys per tile (head sizes up to 128; the BSEL block size)
constexpr float kLazy = 8.f;  // see the lazy rescale in the tile step
constexpr int kBufferConfig = 0x00020000;  // buffer descriptor word 3 (gfx9 family: raw dwords)
constexpr int kNonTemporal = 2;            // cache-policy bit of a buffer load: non-temporal

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max over lanes l and l ^ 32 (the two halves of the wave)
__device__ __forceinline__ float max_halves(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Head size 256 runs 4 waves (one per SIMD, so that each wave can hold 32 rows' O accumulators
// of 256 columns, its Q operand and two S blocks): 128 rows per workgroup.  Smaller heads run 8
// waves, 256 rows.
template <int D>
struct PfCfg {
  static constexpr int NW = D > 128 ? 4 : 8;  // waves
  static constexpr int Threads = 64 * NW;
  static constexpr int RowsWG = 32 * NW;      // (query, head) rows per workgroup
  static constexpr int BN = D > 128 ? 32 : kBN;  // keys per tile (256: registers)
  static constexpr int KB = BN / 32;            // 32-key MFMA blocks per tile
  static constexpr int KStr = D + 8;    // K tile row stride (elements): conflict-free ds_read_b128
  // V tile row stride: a transpose read covers 4 rows x 2 column groups per 32 lanes; rows 16
  // dwords apart (mod 64 banks) make it conflict-free
  static constexpr int VStr = D + 32;
  static constexpr int KK = D / 16;     // MFMA steps over d
  static constexpr int DB = D / 32;     // 32-wide d blocks of O
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int LPT = BN * CPR / Threads;  // chunks per thread per tile (each of K and V)
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// bf16 bits of x rounded toward -inf (a lower bound of x; -inf stays -inf).
__device__ __forceinline__ uint16_t bf16_bits_down(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u >> 16) + ((u >> 31) && (u & 0xFFFFu) ? 1u : 0u));
}

// Inverse of float_key.
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// LDS of the BSEL merge: per wave 32 rows x 16 list entries, then kKeptMax kept entries (one
// query's whole union: g x 16 with g up to 32) and 16 selected ids.
constexpr int kKeptMax = 32 * 16;
constexpr int kMergeCandBytes = (kThreads / 64) * 32 * 16 * 8;
constexpr int kMergeBytes = kMergeCandBytes + (kThreads / 64) * (kKeptMax + 8) * 8;

// BSEL epilogue of one wave (32 rows = 32/g whole queries, since g divides 32): normalize every
// row's list with its LSE, then per query keep the best n of the union of its g lists, one
// entry per block (its group maximum), and write them in ascending block order.  The score key
// is the one of the selection kernels: a * scale_log2 - (LSE * log2(e) - C), C an integer per
// query taken from its first head.  cand_all: 32 x 16 entries per wave; kept_all: kKeptMax
// entries plus 16 ints per wave (LDS the tile loop no longer uses).
template <int kSlots>
__device__ __forceinline__ void select_blocks(const PrefillParams& p,
                                              const unsigned long long (&bl)[kSlots],
                                              float lse_row, unsigned long long* cand_all,
                                              unsigned long long* kept_all, int wave, int lane,
                                              int j0, int nq, int t_min, int b, int u) {
  const int rj = lane & 31, h = lane >> 5;
  const int hh = (wave * 32 + rj) % p.g;
  unsigned long long* cand = cand_all + wave * (32 * 16);
  unsigned long long* kept = kept_all + wave * (kKeptMax + 8);
  int* sel = (int*)(kept + kKeptMax);
  const float lse0 = __shfl(lse_row, (rj - hh) + 32 * h, 64);  // first head of this query
  const double l2 = (double)lse_row * 1.4426950408889634;
  const double Cq = rint((double)lse0 * 1.4426950408889634);
  const float delta = (float)(l2 - Cq);
#pragma unroll
  for (int i = 0; i < kSlots; i++) {
    const unsigned long long e = bl[i];
    unsigned long long v = 0ull;  // empty slot
    if ((e >> 32) != 0ull && e != ~0ull) {
      const float sc = __builtin_fmaf(key_float((uint32_t)(e >> 32)), p.scale_log2, -delta);
      v = ((unsigned long long)float_key(sc) << 32) | (e & 0xFFFFFFFFull);
    }
    cand[rj * 16 + kSlots * h + i] = v;
  }
  const int nc = p.g * 16;  // candidates per query
  for (int qw = 0; qw < 32 / p.g; qw++) {
    const int jq = (wave * 32) / p.g + qw;
    if (jq >= nq) break;  // the same for the whole wave
    wave_sync_lds();
    const unsigned long long* cq = cand + qw * nc;
    // one entry per block id: its largest value (equal values: the lowest index)
    for (int c = lane; c < nc; c += 64) {
      const unsigned long long v = cq[c];
      bool keep = v != 0ull;
      for (int o = 0; o < nc; o++) {
        const unsigned long long w = cq[o];
        keep = keep && !(o != c && (uint32_t)w == (uint32_t)v && (w > v || (w == v && o < c)));
      }
      kept[c] = keep ? v : 0ull;
    }
    if (lane < 16) sel[lane] = -1;
    wave_sync_lds();
    // the kept entries are distinct: the best n_take go to sel[] by rank
    const int n_take = min((t_min + jq) / 64 + 1, p.n_blocks);
    for (int c = lane; c < nc; c += 64) {
      const unsigned long long v = kept[c];
      if (v == 0ull) continue;
      int rank = 0;
      for (int o = 0; o < nc; o++) rank += kept[o] > v;
      if (rank < n_take) sel[rank] = (int)(0xFFFFFFFFu - (uint32_t)v);
    }
    wave_sync_lds();
    // ascending block order, -1 padding, count
    const size_t row = ((size_t)b * p.Tq + j0 + jq) * p.Hkv + u;
    if (lane < p.n_blocks) {
      if (lane < n_take) {
        const int id = sel[lane];
        int pos = 0;
        for (int o = 0; o < n_take; o++) pos += sel[o] < id;
        p.blk_idx[row * p.n_blocks + pos] = id;
      } else {
        p.blk_idx[row * p.n_blocks + lane] = -1;
      }
    }
    if (lane == 0) p.blk_cnt[row] = n_take;
  }
}

// 32x32x16 layouts (wave64, lane l, h = l / 32):
//   A[32 x 16]: row l % 32, k = 8h .. 8h + 7;   B[16 x 32]: column l % 32, k = 8h .. 8h + 7
//   C[32 x 32]: column l % 32, register 4g + e holds row 8g + 4h + e (g, e = 0..3)
// TMAX: every row also records its raw logit maximum over each tile (bf16, rounded toward -inf),
// two tiles per 4-byte store.
// PAGED: K and V are page pools addressed through the block table; a page holds whole tiles,
// so only each tile's first row changes (one scalar table read per tile).
template <int D, bool BSEL, bool TMAX = false, bool PAGED = false>
__global__ __launch_bounds__(PfCfg<D>::Threads, 1) void pf_attn_kernel(PrefillParams p) {
  using C = PfCfg<D>;
  static_assert(!BSEL || C::NW == 8, "the block-selection merge assumes 8 waves");
  static_assert(!TMAX || !BSEL, "tile maxima: not with the block selection");

  // K/V tiles; BSEL reuses the same LDS for its merge after the last tile
  constexpr int BN = C::BN, KB = C::KB;
  static_assert(!BSEL || BN == 64, "blocks of one 64-key tile");
  constexpr int kTileBytes = 2 * BN * (C::KStr + C::VStr) * 2;
  constexpr int kSmemBytes = BSEL && kMergeBytes > kTileBytes ? kMergeBytes : kTileBytes;
  __shared__ __attribute__((aligned(16))) unsigned char pf_smem[kSmemBytes];
  uint16_t (*ks)[BN * C::KStr] = reinterpret_cast<uint16_t (*)[BN * C::KStr]>(pf_smem);
  uint16_t (*vs)[BN * C::VStr] =
      reinterpret_cast<uint16_t (*)[BN * C::VStr]>(pf_smem + 2 * BN * C::KStr * 2);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rj = lane & 31, h = lane >> 5;
  const int qpw = C::RowsWG / p.g;  // queries per workgroup
  const int n_qt = (p.Tq + qpw - 1) / qpw;
  // KV head fastest, then query tile (latest, i.e. longest, first), then batch
  const int u = blockIdx.x % p.Hkv;
  const int qt = n_qt - 1 - (int)((blockIdx.x / p.Hkv) % n_qt);
  const int b = blockIdx.x / (p.Hkv * n_qt);
  const int j0 = qt * qpw;
  const int nq = min(qpw, p.Tq - j0);
  const int t_min = (int)p.q_off + j0;  // positions fit in 31 bits
  const int t_max = t_min + nq - 1;

  // this lane's row: column rj of the wave's S^T / O^T blocks
  const int r = wave * 32 + rj;
  const int jq = r / p.g, hh = r % p.g;
  const bool row_ok = jq < nq;
  const int j_row = j0 + (row_ok ? jq : 0);
  const int h_row = u * p.g + hh;
  const int t_row = t_min + jq;
  bf16x8 qb[C::KK];
  {
    const uint16_t* qp = (const uint16_t*)p.q + (((size_t)b * p.Tq + j_row) * p.Hq + h_row) * D;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) {
      u32x4 raw = row_ok ? *(const u32x4*)(qp + 16 * kk + 8 * h) : u32x4{0, 0, 0, 0};
      qb[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  float m_run = -INFINITY;  // running row maximum, log2 domain (scaled)
  float l_s = 0.f, l_c = 0.f;
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; db++)
#pragma unroll
    for (int i = 0; i < 16; i++) oacc[db][i] = 0.f;

  const size_t kv_row_stride = (size_t)p.Hkv * D;
  const size_t b_rows = PAGED ? 0 : (size_t)b * p.Tk;  // a pool has no batch dimension
  const uint16_t* kbase = (const uint16_t*)p.k + (b_rows * p.Hkv + u) * D;
  const uint16_t* vbase = (const uint16_t*)p.v + (b_rows * p.Hkv + u) * D;
  const int n_tiles = (t_max + BN) / BN;  // tiles covering keys 0..t_max

  // K tiles run one tile ahead of V tiles: the step of tile t takes the softmax of S(t), computed
  // in the previous step, while S(t+1) = K(t+1) Q^T runs on the matrix cores, then O += V(t) P(t).
  // K(t) lives in K buffer t & 1 and V(t) in V buffer t & 1.  The step of tile t stores K(t+2)
  // into K(t)'s buffer (last read by the previous step) and V(t+1) into V(t-1)'s buffer; the
  // barrier ending the step publishes both.  Loads past the last tile read clamped rows, and the
  // last step's S(t+1) is never used, so a step has no branch around its loads or MFMAs.
  // Tile loads are raw buffer loads: the descriptor (scalar registers) holds the tile's first
  // row and its number of valid rows (through t_max); rows past them read as zeros without a
  // memory access (the causal mask covers them), so a thread's byte offset inside a tile is a
  // constant and the loop does no address arithmetic.
  const int row_bytes = p.Hkv * D * 2;
  int voff[C::LPT];
#pragma unroll
  for (int i = 0; i < C::LPT; i++) {
    const int c = threadIdx.x + C::Threads * i;
    voff[i] = (c / C::CPR) * row_bytes + (c % C::CPR) * 16;
  }
  auto tile_rsrc = [&](const uint16_t* base, int t) {
    const int valid = max(0, min(BN, t_max + 1 - t * BN));
    const int n_rec = __builtin_amdgcn_readfirstlane(valid * row_bytes);  // uniform: scalar
    size_t row0 = (size_t)t * BN;
    if constexpr (PAGED) {
      // the tile's page (a tile past the last one, read as zeros, takes the last key's page so
      // that the table index stays inside the batch entry's row of the table)
      const int key0 = min(t * BN, t_max);
      int e = p.pages[(size_t)b * p.max_pages + (key0 >> p.page_shift)];
      e = min(max(e, 0), p.n_pages - 1);
      row0 = ((size_t)e << p.page_shift) + (key0 & ((1 << p.page_shift) - 1));
    }
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + row0 * kv_row_stride), 0, n_rec,
                                             kBufferConfig);
  };
  u32x4 kreg[C::LPT], vreg[C::LPT];
  auto load_k = [&](int t) {
    const auto rs = tile_rsrc(kbase, t);
#pragma unroll
    for (int i = 0; i < C::LPT; i++)
      kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], 0, 0));
  };
  auto load_v = [&](int t) {  // V is read once: non-temporal
    const auto rs = tile_rsrc(vbase, t);
#pragma unroll
    for (int i = 0; i < C::LPT; i++)
      vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], 0, kNonTemporal));
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LPT; i++) {
      const int c = threadIdx.x + C::Threads * i;
      const int row = c / C::CPR, ch = c % C::CPR;
      *(u32x4*)(&ks[buf][row * C::KStr + ch * 8]) = kreg[i];
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LPT; i++) {
      const int c = threadIdx.x + C::Threads * i;
      const int row = c / C::CPR, ch = c % C::CPR;
      *(u32x4*)(&vs[buf][row * C::VStr + ch * 8]) = vreg[i];
    }
  };
  // S^T of tile t for the two 32-key blocks: register 4g + e of s[kb] is key 64t + 32kb + 8g + 4h + e
  auto qk = [&](int t, f32x16 (&s)[KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) s[kb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) {  // the two key blocks' chains interleaved
#pragma unroll
      for (int kb = 0; kb < KB; kb++) {
        const bf16x8 ka = *(const bf16x8*)(&ks[t & 1][(32 * kb + rj) * C::KStr + 16 * kk + 8 * h]);
        s[kb] = mfma32(ka, qb[kk], s[kb]);
      }
    }
  };

  // BSEL: this row's best n blocks as (order-preserving raw maximum << 32 | ~block id); lane
  // half h holds list slots 8h .. 8h+7.  An empty slot holds its own slot number (distinct, and
  // below every real entry, whose upper half is never 0); slots past n_blocks hold ~0 and are
  // never replaced.  thr = the list minimum (slot 0 at first), the same in both halves.
  constexpr int kSlots = 8;
  unsigned long long bl[BSEL ? kSlots : 1];
  unsigned long long thr = 0ull;
  if constexpr (BSEL) {
#pragma unroll
    for (int i = 0; i < kSlots; i++) {
      const int slot = kSlots * h + i;
      bl[i] = slot < p.n_blocks ? (unsigned long long)slot : ~0ull;
    }
  }

  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  load_k(1);
  store_k(1);
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0);  // Q loads done here, not inside the loop
  f32x16 sa[KB], sb[KB];
  qk(0, sa);
  __syncthreads();  // the first step rewrites K buffer 0

  // The step of tile t: S(t) in sc, S(t+1) into sn.  MASK: tile t reaches past the workgroup's
  // first query position.
  float tmx_last = -INFINITY;  // TMAX: the row maximum of the last tile stepped
  auto step = [&](int t, f32x16 (&sc)[KB], f32x16 (&sn)[KB], auto mask_tag)
                  __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    load_k(t + 2);
    load_v(t + 1);
    const int key0 = t * BN;
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int key = key0 + 32 * kb + 8 * (i / 4) + 4 * h + (i % 4);
          sc[kb][i] = (row_ok && key <= t_row) ? sc[kb][i] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sc[kb][i], sc[kb][i + 1]));
    mx = max_halves(mx);
    if constexpr (TMAX) tmx_last = mx;
    if constexpr (BSEL) {
      // block t = this tile: replace the list minimum when the tile's maximum beats it (equal
      // maxima keep the earlier block); both halves of the row take the same branch
      const unsigned long long cand =
          ((unsigned long long)float_key(mx) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)t);
      if (row_ok && mx != -INFINITY && cand > thr) {
#pragma unroll
        for (int i = 0; i < kSlots; i++) bl[i] = bl[i] == thr ? cand : bl[i];
        unsigned long long m = bl[0];
#pragma unroll
        for (int i = 1; i < kSlots; i++) m = bl[i] < m ? bl[i] : m;
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)m, (uint32_t)m, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(m >> 32), (uint32_t)(m >> 32), false, false);
        const unsigned long long m0 = ((unsigned long long)hi[0] << 32) | lo[0];
        const unsigned long long m1 = ((unsigned long long)hi[1] << 32) | lo[1];
        thr = m0 < m1 ? m0 : m1;
      }
    }
    // Lazy rescale: the exponent reference m_run moves only when a row maximum passes it by more
    // than kLazy (log2 units); otherwise p = 2^(s - m_run) <= 2^kLazy, exact in fp32 and bf16, and
    // O, l and the LSE refer to m_run consistently.
    const float m_cand = mx * p.scale_log2;
    if (__ballot(m_cand > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
      l_s *= alpha;
      l_c *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; db++) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
    bf16x8 pb[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; kb++) {
#pragma unroll
      for (int s2 = 0; s2 < 2; s2++) {
        float x8[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          x8[i] = fast_exp2(__builtin_fmaf(sc[kb][8 * s2 + i], p.scale_log2, -m_use));
          psum += x8[i];
        }
        pb[kb][s2] = pack_bf16x8(x8);
      }
    }
    qk(t + 1, sn);

    // O^T += V^T P^T over four 16-key steps; step (kb, s2) covers keys key0 + 32kb + 16s2 + {4h+e,
    // 8+4h+e}, the order in which pb[kb][s2] holds them
#pragma unroll
    for (int kb = 0; kb < KB; kb++) {
#pragma unroll
      for (int s2 = 0; s2 < 2; s2++) {
        const int kbase_row = 32 * kb + 16 * s2 + 4 * h;
#pragma unroll
        for (int db = 0; db < C::DB; db++) {
          const int c0 = 32 * db + 16 * ((lane >> 4) & 1);
          const uint16_t* a0 = &vs[t & 1][(kbase_row + ((lane & 15) >> 2)) * C::VStr + c0 + 4 * (lane & 3)];
          const bf16x8 va = join_tr(lds_read_tr16(a0), lds_read_tr16(a0 + 8 * C::VStr));
          oacc[db] = mfma32(va, pb[kb][s2], oacc[db]);
        }
      }
    }
    // one matrix instruction between every few vector ones: S(t+1) with the exponentials of
    // S(t), then O += V(t) P(t) with the rest (4 and 2 VALU per MFMA measured best: 3 to 8
    // tried, and no hints at all 5 % slower)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 14; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    kahan_add(l_s, l_c, psum);
    store_k(t & 1);
    store_v((t + 1) & 1);
    __syncthreads();
  };
  // TMAX: write the staged maxima of tiles tile0 .. tile0 + 15 (lane: row lane / 2, tiles
  // tile0 + 8 (lane % 2) .. + 7; the row's slots past its last tile hold values of no tile)
  // TMAX: lanes of the first half write their row's maxima of tiles t, t + 1 as one 4-byte store
  uint16_t* tm_dst = nullptr;
  if constexpr (TMAX) {
    if (h == 0 && row_ok)
      tm_dst = p.tile_max + (((size_t)b * p.Hq + h_row) * p.Tq + j_row) * p.tmax_stride;
  }
  auto put_tmax = [&](int t0, float m0, float m1) {
    if constexpr (TMAX) {
      if (tm_dst)
        *(uint32_t*)(tm_dst + t0) = (uint32_t)bf16_bits_down(m0) | ((uint32_t)bf16_bits_down(m1) << 16);
    }
  };
  // tiles entirely at or before the first query position need no mask.  Two steps per loop
  // trip, so that S(t) always sits in sa for even t and in sb for odd t; a tile without mask
  // may run the masked step (the mask is then a no-op)
  const int n_full = min(n_tiles, (t_min + 1) / BN);
  int t = 0;
  for (; t + 1 < n_full; t += 2) {
    step(t, sa, sb, std::false_type());
    const float m0 = tmx_last;
    step(t + 1, sb, sa, std::false_type());
    put_tmax(t, m0, tmx_last);
  }
  for (; t + 1 < n_tiles; t += 2) {
    step(t, sa, sb, std::true_type());
    const float m0 = tmx_last;
    step(t + 1, sb, sa, std::true_type());
    put_tmax(t, m0, tmx_last);
  }
  if (t < n_tiles) {
    step(t, sa, sb, std::true_type());
    put_tmax(t, tmx_last, -INFINITY);  // the pair's second slot lies inside the padded row
  }

  // epilogue: normalize and write O and LSE
  // lanes l and l ^ 32 hold the row's sums over different keys (with the same maximum)
  double ld = (double)l_s - (double)l_c;
  ld += __shfl_xor(ld, 32, 64);
  const float lse_row = ld > 0.0 ? (float)(((double)m_run + log2(ld)) * kLn2) : -INFINITY;
  if constexpr (BSEL)
    select_blocks(p, bl, lse_row, (unsigned long long*)pf_smem,
                  (unsigned long long*)(pf_smem + kMergeCandBytes), wave, lane, j0, nq, t_min, b, u);
  if (!row_ok) return;
  const float inv = ld > 0.0 ? (float)(1.0 / ld) : 0.f;
  const size_t orow = (((size_t)b * p.Tq + j_row) * p.Hq + h_row) * D;
#pragma unroll
  for (int db = 0; db < C::DB; db++) {
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const size_t ooff = orow + 32 * db + 8 * g + 4 * h;
      const f32x4 o4 = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                        oacc[db][4 * g + 3] * inv};
      if (p.out_f32) {
        *(f32x4*)((float*)p.o + ooff) = o4;
      } else {
        typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
        u16x4 h4 = {f2bf(o4[0]), f2bf(o4[1]), f2bf(o4[2]), f2bf(o4[3])};
        *(u16x4*)((uint16_t*)p.o + ooff) = h4;
      }
    }
  }
  if (h == 0) p.lse[((size_t)b * p.Hq + h_row) * p.Tq + j_row] = lse_row;
}

}  // namespace

int prefill_tile_keys(int head_dim) { return head_dim == 256 ? PfCfg<256>::BN : PfCfg<128>::BN; }

hipError_t launch_prefill_attn(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const int rows_wg = head_dim == 256 ? PfCfg<256>::RowsWG : PfCfg<128>::RowsWG;
  if (rows_wg % p.g) return hipErrorInvalidValue;
  const int qpw = rows_wg / p.g;
  const int n_qt = (p.Tq + qpw - 1) / qpw;
  const dim3 grid(p.B * p.Hkv * n_qt);
  const bool bsel = p.blk_idx != nullptr;
  if (bsel && (p.n_blocks < 1 || p.n_blocks > 16 || 32 % p.g || head_dim > 128))
    return hipErrorInvalidValue;
  // tile maxima: head sizes up to 128 (at 256 the kernel has no registers to spare: the maxima
  // cost a fifth of its time), not with the block selection
  if (p.tile_max) {
    if (bsel || p.pages || head_dim > 128 || p.tmax_stride % 16 || p.tmax_stride < (p.Tk + kBN - 1) / kBN)
      return hipErrorInvalidValue;
    if (head_dim == 128) pf_attn_kernel<128, false, true><<<grid, kThreads, 0, stream>>>(p);
    else pf_attn_kernel<64, false, true><<<grid, kThreads, 0, stream>>>(p);
    return hipGetLastError();
  }
  if (p.pages) {  // plain attention only; pages hold whole tiles
    if (bsel || (1 << p.page_shift) < prefill_tile_keys(head_dim) || p.page_shift > 20 ||
        p.max_pages < 1 || p.n_pages < 1)
      return hipErrorInvalidValue;
    if (head_dim == 256)
      pf_attn_kernel<256, false, false, true><<<grid, PfCfg<256>::Threads, 0, stream>>>(p);
    else if (head_dim == 128)
      pf_attn_kernel<128, false, false, true><<<grid, kThreads, 0, stream>>>(p);
    else
      pf_attn_kernel<64, false, false, true><<<grid, kThreads, 0, stream>>>(p);
    return hipGetLastError();
  }
  if (head_dim == 256) {
    pf_attn_kernel<256, false><<<grid, PfCfg<256>::Threads, 0, stream>>>(p);
  } else if (head_dim == 128) {
    if (bsel) pf_attn_kernel<128, true><<<grid, kThreads, 0, stream>>>(p);
    else pf_attn_kernel<128, false><<<grid, kThreads, 0, stream>>>(p);
  } else {
    if (bsel) pf_attn_kernel<64, true><<<grid, kThreads, 0, stream>>>(p);
    else pf_attn_kernel<64, false><<<grid, kThreads, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace hs
