// attn_rows.hip -- row-attention kernel: softmax attention of up to 16 packed (query, head) rows
// of one KV head over a key list, split across workgroups and waves, plus the split combine.
//
// One kernel serves four uses that differ only in where the keys come from:
//   * full-attention decode / short query blocks (contiguous positions 0..t)
//     [P2 "Extracting block scores from exact attention": a = q.k/sqrt(d), p = softmax, o = sum p v];
//   * HySparse2 token-sparse layers: keys = the shared index set of (b, t, u) read from the full
//     layer's K, V [P2 "Cross-layer KV cache reuse" gather equations; P1 section 4.2];
//   * HySparse block-sparse branch: keys = whole 64-token blocks, causal inside a block that
//     crosses t [P2 "Same query, two memories"; P2 engineering constraint 4];
//   * HySparse sliding-window branch over the layer's own K', V' (contiguous t-w+1..t)
//     [P2 "Same query, two memories", SWA equation].
// Gathering is index-driven straight from HBM into registers (K) and LDS (V): no gathered copy
// of K/V is ever written back [P2 engineering constraint 3 warns that gather-to-temp doubles
// the traffic].
//
// Layout on the MFMA (v_mfma_f32_16x16x32_bf16, see hs_device.h):
//   S^T = K Q^T : A = 16 keys x d from HBM, B = Q^T kept in registers  -> lane (row n, group j)
//                 holds S[row n][keys 4j..4j+3] of each 16-key block.
//   O^T += V^T P^T : B = P^T is exactly the S^T output (no shuffle), A = V^T read from a
//                 row-major LDS tile with ds_read_b64_tr_b16.
// Every per-row statistic (running max, sum) lives in the 4 lanes of that row.
#include <type_traits>

#include "hs_device.h"
#include "hs_kernels.h"

namespace hs {
namespace {

constexpr int kStep = 32;  // keys per wave step
constexpr int kXcds = 8;   // accelerator complex dies of MI355X (workgroups go round-robin)
constexpr int kMaxListEntries = 2048;  // list-mode entries staged per workgroup (64 steps)

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not wait for this
// wave's global stores to be acknowledged (the stored logits need no ordering before the merge).
__device__ __forceinline__ void workgroup_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// NW: waves per workgroup (4, or 8 for unsplit key lists of few row-sets)
template <int D, bool F32, int NW>
struct RaCfg {
  static constexpr int kWaves = NW;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kTPR = kThreads / 16;  // merge threads per row
  static constexpr int kCPT = D / kTPR;       // merge columns per thread
  // A merge thread's columns come in chunks of up to 4 consecutive ones, the chunks kTPR * kChunk
  // columns apart: the kTPR threads of a row then read and write contiguous 16-byte pieces
  // (conflict-free in LDS, coalesced in memory).
  static constexpr int kChunk = kCPT < 4 ? kCPT : 4;
  static constexpr int kOStride = D + 4;  // merge buffer row stride (floats)
  __device__ static int col(int lr, int c) {
    return ((c / kChunk) * kTPR + lr) * kChunk + c % kChunk;
  }
  static constexpr int kElem = F32 ? 4 : 2;
  static constexpr int kVStride = D + (F32 ? 4 : 16);  // LDS row stride (elements), padded
  static constexpr int kChunksPerRow = D * kElem / 16;
  static constexpr int kVLoads = kStep * kChunksPerRow / 64;  // 16-byte V chunks per lane
  static constexpr int kVTileBytes = kStep * kVStride * kElem;
  static constexpr int kCombineBytes =
      kWaves * 16 * kOStride * 4 + kWaves * 16 * 4 + kWaves * 16 * 8;
  static constexpr int kSmem =
      (kWaves * kVTileBytes > kCombineBytes ? kWaves * kVTileBytes : kCombineBytes);
};

// Logits kept by the full-attention pass are staged per wave in LDS and written out every
// kLogitSteps steps: a global store issued between the loads of the software pipeline delays the
// wait for every later load until the store is acknowledged (the vector memory counter is in
// order), so few, large store bursts cost far less than two small stores per step.
constexpr int kLogitSteps = 4;
constexpr int kLogitRow = kLogitSteps * kStep + 4;  // floats per staged row (padded)
constexpr int kLogitWaveBytes = 16 * kLogitRow * 4;

// Position of key-list entry e (-1: none).  The list entry is read whether or not e is below the
// list's length L (every entry below idx_cap, or idx_cap blocks, lies inside the caller's index
// array), so that the entry loads need not wait for the count load.
template <int SRC>
__device__ __forceinline__ int entry_pos(const RowAttnParams& p, int e, int L, long long lo,
                                         long long t_last, const int32_t* list) {
  if (SRC == SRC_RANGE || SRC == SRC_WINDOW) return e < L ? (int)(lo + e) : -1;
  if (SRC == SRC_TOKEN) {
    const int x = e < p.idx_cap ? list[e] : -1;
    return (e < L && x >= 0 && x <= t_last) ? x : -1;
  }
  const int eb = e / p.block;
  const int blk = eb < p.idx_cap ? list[eb] : -1;
  if (e >= L || blk < 0 || (long long)blk > t_last / p.block) return -1;
  const long long x = (long long)blk * p.block + e % p.block;
  return x <= t_last ? (int)x : -1;
}

// Result of one pass over a key source, as held by the merge thread of row r, columns
// RaCfg::col(lr, c), c < CPT (r = threadIdx.x / TPR, lr = threadIdx.x % TPR): the row maximum
// M (log2 domain), the row sum L relative to M and the unnormalized output columns.
template <int CPT>
struct PassOut {
  float M;
  double L;
  float ov[CPT];
};

// One split of one row-set over one key source (K, V given explicitly so that the gated layer
// can run its window branch over K', V' in the same workgroup).  Ends with the four waves
// merged; `smem` and `pos_all` are free again once the caller has synchronized.  LOGITS (range
// mode only): every lane also stores the raw dot products q.k it computed to p.logits.
// PAGED (range and list modes): K and V are page pools [n_pages, page_size, Hkv, d] addressed
// through the block table; `row_all` holds the split's physical rows (list modes).  The window
// source reads a ring of p.ring slots (position t at slot t % ring) when p.ring > 0.
template <int D, bool F32, int SRC, int NW, bool LOGITS = false, bool PAGED = false>
__device__ __forceinline__ void attend_pass(const RowAttnParams& p, const void* kmat,
                                            const void* vmat, int split, int steps_per_split,
                                            int b, int u, int hc, int j0, int nq,
                                            unsigned char* smem, int* pos_all, int* row_all,
                                            PassOut<RaCfg<D, F32, NW>::kCPT>& out) {
  using Cfg = RaCfg<D, F32, NW>;
  constexpr int kWaves = NW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rn = lane & 15;   // MFMA row / column index of this lane
  const int jg = lane >> 4;   // lane group 0..3
  const int hcn = min(p.hpc, p.g - hc * p.hpc);  // heads of chunk hc (the last may be short)
  const int nrows = nq * hcn;  // a set: nq queries x the heads of head chunk hc
  const long long t_first = p.q_off + j0;
  const long long t_last = p.q_off + j0 + nq - 1;

  int L;
  long long lo = 0;
  const int32_t* list = nullptr;
  if (SRC == SRC_RANGE || SRC == SRC_WINDOW) {
    lo = (SRC == SRC_WINDOW) ? (t_first - p.window + 1 > 0 ? t_first - p.window + 1 : 0) : 0;
    L = (int)(t_last - lo + 1);
  } else {
    const long long row = ((long long)b * p.Tq + j0) * p.Hkv + u;
    list = p.idx + row * p.idx_cap;
    int c = p.cnt[row];
    c = c < 0 ? 0 : (c > p.idx_cap ? p.idx_cap : c);
    L = (SRC == SRC_TOKEN) ? c : c * p.block;
  }

  // this lane's row (for Q, masks and statistics)
  const bool row_ok = rn < nrows;
  const int jq = row_ok ? rn / hcn : 0;
  const int hh = hc * p.hpc + (row_ok ? rn % hcn : 0);
  const long long t_row = p.q_off + j0 + jq;
  const int h = u * p.g + hh;
  const long long lo_row = (SRC == SRC_WINDOW) ? t_row - p.window + 1 : 0;

  const size_t kv_row_stride = (size_t)p.Hkv * D;  // elements between consecutive positions
  const size_t kv_base = ((size_t)b * p.Tk * p.Hkv + u) * D;

  // ---- Q^T operand, resident for the whole kernel ----
  constexpr int KK = F32 ? D / 4 : D / 32;  // MFMA steps over d
  bf16x8 qb[F32 ? 1 : KK];
  float qf[F32 ? KK : 1];
  {
    const size_t qoff = (((size_t)b * p.Tq + (j0 + jq)) * p.Hq + h) * D;
    if constexpr (!F32) {
      const uint16_t* qp = (const uint16_t*)p.q + qoff;
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        u32x4 raw = row_ok ? *(const u32x4*)(qp + 32 * kk + 8 * jg) : u32x4{0, 0, 0, 0};
        qb[kk] = __builtin_bit_cast(bf16x8, raw);
      }
    } else {
      const float* qp = (const float*)p.q + qoff + jg * KK;
#pragma unroll
      for (int s = 0; s < KK; s++) qf[s] = row_ok ? qp[s] : 0.f;
    }
  }

  // ---- running softmax state (log2 domain) and output accumulators O^T ----
  float m_run = -INFINITY;
  float l_s = 0.f, l_c = 0.f;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_steps = (L + kStep - 1) / kStep;
  const int step_begin = split * steps_per_split;
  const int step_end = min(step_begin + steps_per_split, n_steps);
  unsigned char* vtile = smem + wave * Cfg::kVTileBytes;

  // LOGITS: this wave's staging rows [16][kLogitRow] behind the V tiles, the number of steps
  // staged so far and the first step of the current batch
  float* lbuf = nullptr;
  int l_count = 0, l_base = 0;
  if constexpr (LOGITS) {
    static_assert(SRC == SRC_RANGE, "logits are written by the full-attention pass only");
    lbuf = (float*)(smem + kWaves * Cfg::kVTileBytes + wave * kLogitWaveBytes);
  }
  // Write the n staged steps l_base, l_base + kWaves, ... of this wave to the logit array
  // [B, Tq, Hq, Tk]: 128-byte pieces (32 keys of one row), 16 bytes per lane.
  auto flush_logits = [&](int n) {
    wave_lds_sync();  // staged values written by every lane
    const int chunks = nrows * n * 8;
    for (int c = lane; c < chunks; c += 64) {
      const int r = c / (n * 8), li = (c / 8) % n, qd = c % 8;
      const int e0 = (l_base + li * kWaves) * kStep + 4 * qd;  // range mode: entry = position
      float* dst = p.logits + (((size_t)b * p.Tq + (j0 + r / hcn)) * p.Hq + u * p.g +
                                hc * p.hpc + r % hcn) *
                                  (size_t)p.Tk + e0;
      const f32x4 val = *(const f32x4*)(lbuf + r * kLogitRow + li * kStep + 4 * qd);
      if (p.logits_vec && e0 + 3 < L) {
        *(f32x4*)dst = val;
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (e0 + e < L) dst[e] = val[e];
      }
    }
    wave_lds_sync();  // staging rows free again
  };

  // Positions of this split's key-list entries.  List modes stage them in LDS once (so the
  // K/V loads of the next step can be issued without waiting on an index load); range modes
  // compute them.  PAGED: list modes also stage each entry's physical row; the range mode
  // stages the physical page of every logical page the split touches.
  constexpr bool kList = (SRC == SRC_TOKEN || SRC == SRC_BLOCK);
  static_assert(!PAGED || SRC == SRC_RANGE || kList, "the window source is never paged");
  const int pg_shift = PAGED ? __ffs(p.page_size) - 1 : 0;
  const int32_t* table = PAGED ? p.pages + (size_t)b * p.max_pages : nullptr;
  auto phys_page = [&](int logical) -> int {
    const int e = table[logical];
    return e < 0 ? 0 : (e >= p.n_pages ? p.n_pages - 1 : e);  // stays inside the pool
  };
  int first_page = 0;
  if constexpr (kList) {
    // the split's whole entry range (its length does not depend on the count, so the entry
    // loads are issued together with the count load); entries past the list read as -1
    const int n_e = steps_per_split * kStep < kMaxListEntries ? steps_per_split * kStep
                                                                : kMaxListEntries;
    for (int i = threadIdx.x; i < n_e; i += Cfg::kThreads) {
      const int pos = entry_pos<SRC>(p, step_begin * kStep + i, L, lo, t_last, list);
      pos_all[i] = pos;
      if constexpr (PAGED) {
        const int q = pos < 0 ? 0 : pos;
        row_all[i] = (phys_page(q >> pg_shift) << pg_shift) | (q & (p.page_size - 1));
      }
    }
    __syncthreads();
  } else if constexpr (PAGED) {
    if (step_begin < step_end) {
      first_page = (int)((lo + (long long)step_begin * kStep) >> pg_shift);
      const int last_page = (int)((lo + min((long long)step_end * kStep, (long long)L) - 1) >> pg_shift);
      for (int i = threadIdx.x; i <= last_page - first_page; i += Cfg::kThreads)
        pos_all[i] = phys_page(first_page + i);
    }
    __syncthreads();
  }
  // element offset of key entry i of a step (position pos >= 0, or -1: any valid row) in K / V
  auto kv_off = [&](int step, int i, int pos) -> size_t {
    if constexpr (PAGED && kList) {
      return ((size_t)row_all[(step - step_begin) * kStep + i] * p.Hkv + u) * D;
    } else if constexpr (PAGED) {
      const int q = pos < 0 ? 0 : pos;  // past the end: any staged row
      const int pg = (q >> pg_shift) - first_page;
      const size_t row = ((size_t)pos_all[pg < 0 ? 0 : pg] << pg_shift) |
                         (size_t)(q & (p.page_size - 1));
      return (row * p.Hkv + u) * D;
    } else if constexpr (SRC == SRC_WINDOW) {
      if (pos < 0) pos = 0;
      if (p.ring > 0) return (((size_t)b * p.ring + pos % p.ring) * p.Hkv + u) * D;
      return kv_base + (size_t)pos * kv_row_stride;
    } else {
      if (pos < 0) pos = 0;
      return kv_base + (size_t)pos * kv_row_stride;
    }
  };
  auto pos_of = [&](int step, int i) -> int {
    if constexpr (kList) {
      return pos_all[(step - step_begin) * kStep + i];
    } else {
      const int e = step * kStep + i;
      return e < L ? (int)(lo + e) : -1;
    }
  };

  // Software pipeline: the K and V rows of a wave's next step are requested before the current
  // step is computed.  K goes to registers in MFMA operand layout, V to registers and then to
  // this wave's LDS tile.
  constexpr int VL = Cfg::kVLoads;
  using KReg = typename std::conditional<F32, float, u32x4>::type;
  auto load_step = [&](int step, KReg (&k0)[KK], KReg (&k1)[KK], u32x4 (&vr)[VL]) {
    const int pk0 = pos_of(step, rn), pk1 = pos_of(step, 16 + rn);
    const size_t ko0 = kv_off(step, rn, pk0), ko1 = kv_off(step, 16 + rn, pk1);
    if constexpr (!F32) {
      const uint16_t* kp0 = (const uint16_t*)kmat + ko0 + 8 * jg;
      const uint16_t* kp1 = (const uint16_t*)kmat + ko1 + 8 * jg;
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        k0[kk] = *(const u32x4*)(kp0 + 32 * kk);
        k1[kk] = *(const u32x4*)(kp1 + 32 * kk);
      }
    } else {
      const float* kp0 = (const float*)kmat + ko0 + jg * KK;
      const float* kp1 = (const float*)kmat + ko1 + jg * KK;
#pragma unroll
      for (int s2 = 0; s2 < KK; s2++) {
        k0[s2] = kp0[s2];
        k1[s2] = kp1[s2];
      }
    }
#pragma unroll
    for (int n = 0; n < VL; n++) {
      const int c = n * 64 + lane;
      const int e = c / Cfg::kChunksPerRow, qc = c % Cfg::kChunksPerRow;
      const int pv = pos_of(step, e);
      const unsigned char* vp = (const unsigned char*)vmat + kv_off(step, e, pv) * Cfg::kElem + qc * 16;
      vr[n] = ld_stream(vp);
    }
  };

  // One 32-key step of this wave on K rows (ka0, ka1) and V rows (va) already in registers.
  auto compute_step = [&](int step, const KReg (&ka0)[KK], const KReg (&ka1)[KK],
                          const u32x4 (&va)[VL]) {
    // V rows of this step -> LDS tile (row-major [key][d], padded rows)
#pragma unroll
    for (int n = 0; n < VL; n++) {
      const int c = n * 64 + lane;
      const int e = c / Cfg::kChunksPerRow, qc = c % Cfg::kChunksPerRow;
      *(u32x4*)(vtile + (e * Cfg::kVStride) * Cfg::kElem + qc * 16) = va[n];
    }

    // S^T = K Q^T for the two 16-key blocks
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (!F32) {
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        sacc[0] = mfma_bf16(__builtin_bit_cast(bf16x8, ka0[kk]), qb[kk], sacc[0]);
        sacc[1] = mfma_bf16(__builtin_bit_cast(bf16x8, ka1[kk]), qb[kk], sacc[1]);
      }
    } else {
#pragma unroll
      for (int s2 = 0; s2 < KK; s2++) {
        sacc[0] = mfma_f32(ka0[s2], qf[s2], sacc[0]);
        sacc[1] = mfma_f32(ka1[s2], qf[s2], sacc[1]);
      }
    }

    if constexpr (LOGITS) {
      // lane (row rn, group jg) holds the dot products of entries 16 kb + 4 jg + e of the step;
      // keys past a row's own position are written as well (the caller ignores them)
      const int slot = l_count % kLogitSteps;
      if (slot == 0) l_base = step;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
        *(f32x4*)(lbuf + rn * kLogitRow + slot * kStep + 16 * kb + 4 * jg) = sacc[kb];
      l_count++;
      if (slot == kLogitSteps - 1) flush_logits(kLogitSteps);
    }

    // scale to the log2 domain and mask
    float sv[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int pos = pos_of(step, 16 * kb + 4 * jg + e);
        const bool ok = row_ok && pos >= 0 && pos <= t_row && pos >= lo_row;
        const float x = ok ? sacc[kb][e] * p.scale_log2 : -INFINITY;
        sv[kb][e] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = max4groups(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
    float pv8[8];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float pe = fast_exp2(sv[kb][e] - m_use);
        pv8[4 * kb + e] = pe;
        psum += pe;
      }
    l_s *= alpha;
    l_c *= alpha;
    kahan_add(l_s, l_c, psum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 16; db++) oacc[db] *= alpha;

    wave_lds_sync();  // V tile written by every lane of this wave

    if constexpr (!F32) {
      const bf16x8 pb = pack_bf16x8(pv8);
      const uint16_t* vt = (const uint16_t*)vtile;
#pragma unroll
      for (int db = 0; db < D / 16; db++) {
        const uint16_t* a0 = vt + (4 * jg + (rn >> 2)) * Cfg::kVStride + 16 * db + 4 * (rn & 3);
        const uint16_t* a1 = a0 + 16 * Cfg::kVStride;
        const bf16x8 vop = join_tr(lds_read_tr16(a0), lds_read_tr16(a1));
        oacc[db] = mfma_bf16(vop, pb, oacc[db]);
      }
    } else {
      const float* vt = (const float*)vtile;
#pragma unroll
      for (int db = 0; db < D / 16; db++)
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float vop = vt[(16 * kb + 4 * jg + e) * Cfg::kVStride + 16 * db + rn];
            oacc[db] = mfma_f32(vop, pv8[4 * kb + e], oacc[db]);
          }
    }
    wave_lds_sync();  // tile reads done before the next step overwrites it
  };

  // The loop always prefetches (its last step is peeled off below): a conditional prefetch
  // would make the compiler wait for the first prefetched load before every step.
  KReg ka0[KK], ka1[KK];
  u32x4 va[VL];
  int step = step_begin + wave;
  if (step < step_end) load_step(step, ka0, ka1, va);
  for (; step + kWaves < step_end; step += kWaves) {
    KReg kn0[KK], kn1[KK];
    u32x4 vn[VL];
    load_step(step + kWaves, kn0, kn1, vn);
    compute_step(step, ka0, ka1, va);
#pragma unroll
    for (int kk = 0; kk < KK; kk++) {
      ka0[kk] = kn0[kk];
      ka1[kk] = kn1[kk];
    }
#pragma unroll
    for (int n = 0; n < VL; n++) va[n] = vn[n];
  }
  if (step < step_end) compute_step(step, ka0, ka1, va);
  if constexpr (LOGITS) {
    if (l_count % kLogitSteps) flush_logits(l_count % kLogitSteps);
  }

  // ---- merge the waves of this workgroup ----
  // (rows kOStride = D + 4 floats apart: the 16 rows' 16-byte writes of one column block fall in
  // distinct bank groups)
  workgroup_lds_sync();
  constexpr int OS = Cfg::kOStride;
  float* cO = (float*)smem;                     // [kWaves][16][OS]
  float* cM = cO + kWaves * 16 * OS;            // [kWaves][16]
  double* cL = (double*)(cM + kWaves * 16);     // [kWaves][16]
#pragma unroll
  for (int db = 0; db < D / 16; db++) *(f32x4*)&cO[(wave * 16 + rn) * OS + 16 * db + 4 * jg] = oacc[db];
  double ld = (double)l_s - (double)l_c;
  ld += __shfl_xor(ld, 16, 64);
  ld += __shfl_xor(ld, 32, 64);
  if (jg == 0) {
    cM[wave * 16 + rn] = m_run;
    cL[wave * 16 + rn] = ld;
  }
  workgroup_lds_sync();

  constexpr int CPT = Cfg::kCPT;
  const int r = threadIdx.x / Cfg::kTPR;
  const int lr = threadIdx.x % Cfg::kTPR;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; w++) M = fmaxf(M, cM[w * 16 + r]);
  double Ls = 0.0;
  float f[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; w++) {
    const float mw = cM[w * 16 + r];
    f[w] = (mw == -INFINITY) ? 0.f : (float)exp2((double)mw - (double)M);
    Ls += (mw == -INFINITY) ? 0.0 : exp2((double)mw - (double)M) * cL[w * 16 + r];
  }
#pragma unroll
  for (int c = 0; c < CPT; c++) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) acc += f[w] * cO[(w * 16 + r) * OS + Cfg::col(lr, c)];
    out.ov[c] = acc;
  }
  out.M = M;
  out.L = Ls;
}

// LDS bytes of a row-kernel workgroup besides its position lists.
template <int D, bool F32, int NW, bool LOGITS>
constexpr int row_attn_smem_bytes() {
  using Cfg = RaCfg<D, F32, NW>;
  // LOGITS: the logit staging rows of every wave follow the V tiles
  return LOGITS && NW * (Cfg::kVTileBytes + kLogitWaveBytes) > Cfg::kSmem
             ? NW * (Cfg::kVTileBytes + kLogitWaveBytes)
             : Cfg::kSmem;
}

// One workgroup of a row-kernel launch: workgroup `bid` of `nblocks`, with the LDS arrays of the
// calling kernel (smem: row_attn_smem_bytes; pos_all, row_all: kMaxListEntries ints).
// GATED: the HySparse sparse layer in one workgroup when neither branch is split -- the block
// (or token) branch over K, V, then the sliding-window branch over K', V' (p.k2, p.v2), each
// normalized on its own and weighted by its sigmoid gate [P2 "Same query, two memories"].
template <int D, bool F32, int SRC, bool GATED, int NW, bool LOGITS, bool PAGED>
__device__ __forceinline__ void row_attn_wg(const RowAttnParams& p, int bid, int nblocks,
                                            unsigned char* smem, int* pos_all, int* row_all) {
  using Cfg = RaCfg<D, F32, NW>;

  // Workgroup order: KV head fastest, then split, then (batch, query chunk), so that the
  // workgroups reading the same positions of the Hkv interleaved heads run together (whole
  // [Hkv, d] rows of K and V are then consumed close in time).  query_major (index lists of
  // many queries): query fastest, so that the workgroups resident at one time gather from the
  // K and V of one (batch entry, KV head), which then stay in the last-level cache.
  // Head chunks (groups of more than 16 heads: 16 heads per set) of one key range read the
  // same K and V rows: they are placed on the same XCD (consecutive workgroup ids go round-robin
  // over the 8 XCDs, each with its own L2), so that the rows come from HBM once.
  int hc = 0, x = bid;
  if (p.cpq > 1) {
    const int n8 = kXcds * p.cpq;
    const int full = (nblocks / n8) * n8;
    if (bid < full) {
      const int grp = bid / n8, within = bid % n8;
      hc = within / kXcds;
      x = grp * kXcds + within % kXcds;
    } else {
      hc = (bid - full) % p.cpq;
      x = full / p.cpq + (bid - full) / p.cpq;
    }
  }
  int u, split, sq, b;
  if (p.query_major) {  // query fastest, then split, then (batch, KV head)
    sq = x % p.sets_per_bu;
    split = (x / p.sets_per_bu) % p.n_split;
    const int bu = x / (p.sets_per_bu * p.n_split);
    u = bu % p.Hkv;
    b = bu / p.Hkv;
  } else {
    u = x % p.Hkv;
    split = (x / p.Hkv) % p.n_split;
    const int bq = x / (p.Hkv * p.n_split);
    sq = bq % p.sets_per_bu;
    b = bq / p.sets_per_bu;
  }
  const int set = ((b * p.Hkv + u) * p.sets_per_bu + sq) * p.cpq + hc;
  const int j0 = sq * p.q_per_set;
  const int nq = min(p.q_per_set, p.Tq - j0);
  const int hcn = min(p.hpc, p.g - hc * p.hpc);  // heads of chunk hc (the last may be short)
  const int nrows = nq * hcn;

  constexpr int CPT = Cfg::kCPT;  // columns per merge thread
  PassOut<CPT> a;
  attend_pass<D, F32, SRC, NW, LOGITS, PAGED>(p, p.k, p.v, split, p.steps_per_split, b, u, hc,
                                              j0, nq, smem, pos_all, row_all, a);

  const int r = threadIdx.x / Cfg::kTPR;
  const int lr = threadIdx.x % Cfg::kTPR;
  const int jr = j0 + r / hcn;
  const int hr = u * p.g + hc * p.hpc + r % hcn;
  const size_t orow = ((size_t)b * p.Tq + jr) * p.Hq + hr;  // (b, t, h) of this thread's row
  float res[CPT];
  float lse_row = -INFINITY;
  if constexpr (GATED) {
    __syncthreads();  // merge buffers are reused by the window pass
    PassOut<CPT> w;
    attend_pass<D, F32, SRC_WINDOW, NW>(p, p.k2, p.v2, 0, 1 << 30, b, u, hc, j0, nq, smem,
                                        pos_all, row_all, w);
    if (r >= nrows) return;
    if (p.gate_ch) {  // per-channel gates: (zG_c, zL_c) and the output gate of column c
      const float* zg = p.gate + orow * 2 * D;
      const float* og = p.out_gate ? p.out_gate + orow * D : nullptr;
      const RowNorm ng = row_norm(a.M, a.L, p.sink, hr, 1.0);
      const RowNorm nl = row_norm(w.M, w.L, p.sink2, hr, 1.0);
#pragma unroll
      for (int c = 0; c < CPT; c++) {
        const int col = Cfg::col(lr, c);
        const float go = og ? sigmoid_f(og[col]) : 1.f;
        res[c] = go * (a.ov[c] * ng.factor * sigmoid_f(zg[col]) +
                       w.ov[c] * nl.factor * sigmoid_f(zg[D + col]));
      }
      lse_row = ng.lse;
    } else {
      const float* z = p.gate + orow * 2;
      const double og = out_gate_of(p.out_gate, orow);
      const double sg = 1.0 / (1.0 + exp(-(double)z[0]));
      const double sl = 1.0 / (1.0 + exp(-(double)z[1]));
      const RowNorm ng = row_norm(a.M, a.L, p.sink, hr, sg * og);
      const RowNorm nl = row_norm(w.M, w.L, p.sink2, hr, sl * og);
#pragma unroll
      for (int c = 0; c < CPT; c++) res[c] = a.ov[c] * ng.factor + w.ov[c] * nl.factor;
      lse_row = ng.lse;
    }
  } else {
    if (!p.final_direct) {
      const size_t n_sets = (size_t)p.B * p.Hkv * p.sets_per_bu * p.cpq;
      const size_t prow = ((size_t)split * n_sets + set) * 16 + r;
      if (r < nrows) {
        if (lr == 0) {
          p.part_m[prow] = a.M;
          p.part_l[prow] = a.L;
        }
#pragma unroll
        for (int c = 0; c < CPT; c++) p.part_o[prow * D + Cfg::col(lr, c)] = a.ov[c];
      }
      return;
    } else {
      if (r >= nrows) return;
      if (p.gate_ch && p.out_gate) {  // per-channel output gate
        const RowNorm n = row_norm(a.M, a.L, p.sink, hr, 1.0);
        const float* og = p.out_gate + orow * D;
#pragma unroll
        for (int c = 0; c < CPT; c++)
          res[c] = a.ov[c] * n.factor * sigmoid_f(og[Cfg::col(lr, c)]);
        lse_row = n.lse;
      } else {
        const RowNorm n = row_norm(a.M, a.L, p.sink, hr, out_gate_of(p.out_gate, orow));
#pragma unroll
        for (int c = 0; c < CPT; c++) res[c] = a.ov[c] * n.factor;
        lse_row = n.lse;
      }
    }
  }
  if (p.out_f32) {
    float* op = (float*)p.o + orow * D;
#pragma unroll
    for (int c = 0; c < CPT; c++) op[Cfg::col(lr, c)] = res[c];
  } else {
    uint16_t* op = (uint16_t*)p.o + orow * D;
#pragma unroll
    for (int c = 0; c < CPT; c++) op[Cfg::col(lr, c)] = f2bf(res[c]);
  }
  if (p.lse && lr == 0) p.lse[((size_t)b * p.Hq + hr) * p.Tq + jr] = lse_row;
}

template <int D, bool F32, int SRC, bool GATED, int NW, bool LOGITS = false, bool PAGED = false>
__global__ __launch_bounds__(64 * NW) void row_attn_kernel(RowAttnParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[row_attn_smem_bytes<D, F32, NW, LOGITS>()];
  __shared__ int pos_all[kMaxListEntries];
  __shared__ int row_all[PAGED && SRC != SRC_RANGE ? kMaxListEntries : 1];
  row_attn_wg<D, F32, SRC, GATED, NW, LOGITS, PAGED>(p, blockIdx.x, gridDim.x, smem, pos_all,
                                                     row_all);
}

// Both branches of a gated sparse layer whose lists are split, in one launch: the first
// n_glob workgroups take the split token / block lists over K, V (pg), the others the sliding
// window over K', V' (pl); all write split partials for the two-branch combine.  One launch
// instead of two: the window branch's workgroups run beside the list branch's instead of after
// them.
template <int D, bool F32, int SRC, int NW, bool PAGED>
__global__ __launch_bounds__(64 * NW) void row_attn_two_kernel(RowAttnParams pg, RowAttnParams pl,
                                                               int n_glob) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[row_attn_smem_bytes<D, F32, NW, false>()];
  __shared__ int pos_all[kMaxListEntries];
  __shared__ int row_all[PAGED ? kMaxListEntries : 1];
  if ((int)blockIdx.x < n_glob)
    row_attn_wg<D, F32, SRC, false, NW, false, PAGED>(pg, blockIdx.x, n_glob, smem, pos_all,
                                                      row_all);
  else
    row_attn_wg<D, F32, SRC_WINDOW, false, NW, false, false>(
        pl, blockIdx.x - n_glob, gridDim.x - n_glob, smem, pos_all, row_all);
}

// ---- split / branch combine ---------------------------------------------------------------
// One workgroup per (row-set, row), q_per_set * hpc rows per set.  Threads = SP split lanes x D/4 column chunks; each thread
// folds every SP-th split of its 4 columns with weights 2^(m_s - M), then the split lanes are
// summed in LDS.  Row sums are combined in fp64.
// BATCHED (more than two splits per thread): the loads of kBatch splits are issued before any
// is used, here and below (a dependent load per split makes the combine a chain of round
// trips); with at most two splits per thread the plain loops, with fewer registers, are faster.
template <int D, bool BATCHED>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int NC = D / 4;         // column chunks of 4
  constexpr int SP = 256 / NC;      // split lanes
  __shared__ float red[SP][D];
  __shared__ double redl[SP];
  const int rps = p.q_per_set * p.hpc;  // rows of a full row-set (the grid has rps per set)
  const int set = blockIdx.x / rps;
  const int r = blockIdx.x % rps;
  const size_t n_sets = gridDim.x / rps;
  const int hc = set % p.cpq;
  const int sq = (set / p.cpq) % p.sets_per_bu;
  const int bu = set / (p.cpq * p.sets_per_bu);
  const int u = bu % p.Hkv;
  const int b = bu / p.Hkv;
  const int j0 = sq * p.q_per_set;
  const int nq = min(p.q_per_set, p.Tq - j0);
  const int hcn = min(p.hpc, p.g - hc * p.hpc);  // heads of chunk hc (the last may be short)
  if (r >= nq * hcn) return;  // whole workgroup leaves together
  const int jr = j0 + r / hcn;
  const int hr = u * p.g + hc * p.hpc + r % hcn;
  const int c = threadIdx.x % NC;
  const int sl = threadIdx.x / NC;

  float out[4] = {0.f, 0.f, 0.f, 0.f};
  double lse0 = -INFINITY;
  const size_t orow = ((size_t)b * p.Tq + jr) * p.Hq + hr;
  const double og = p.gate_ch ? 1.0 : out_gate_of(p.out_gate, orow);
  float og_ch[4] = {1.f, 1.f, 1.f, 1.f};  // per-channel output gate of this thread's columns
  if (p.gate_ch && p.out_gate && threadIdx.x < NC) {
#pragma unroll
    for (int e = 0; e < 4; e++) og_ch[e] = sigmoid_f(p.out_gate[orow * D + 4 * c + e]);
  }
  for (int br = 0; br < p.n_branch; br++) {
    const int ns = p.n_split[br];
    const float* m = p.m[br];
    // row maximum over splits (every thread, redundantly)
    constexpr int kBatch = 8;
    // unbatched: a thread folds at most two splits (sl and sl + SP); their loads are issued
    // before the row maximum is known (a split past the end reads split 0, weighted 0)
    float m2[2];
    f32x4 o2[2];
    double l2[2];
    // batched: the first batch of this thread's splits (sl, sl + SP, ...), likewise loaded
    // before the row maximum
    float mb0[BATCHED ? kBatch : 1];
    f32x4 ob0[BATCHED ? kBatch : 1];
    double lb0[BATCHED ? kBatch : 1];
    if constexpr (BATCHED) {
#pragma unroll
      for (int i = 0; i < kBatch; i++) {
        const int si = sl + i * SP;
        const size_t prow = ((size_t)(si < ns ? si : 0) * n_sets + set) * 16 + r;
        mb0[i] = si < ns ? m[prow] : -INFINITY;
        ob0[i] = *(const f32x4*)(p.po[br] + prow * D + 4 * c);
        lb0[i] = c == 0 ? p.l[br][prow] : 0.0;
      }
    }
    if constexpr (!BATCHED) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int s = sl + i * SP;
        const size_t prow = ((size_t)(s < ns ? s : 0) * n_sets + set) * 16 + r;
        m2[i] = m[prow];
        o2[i] = *(const f32x4*)(p.po[br] + prow * D + 4 * c);
        l2[i] = p.l[br][prow];
        if (s >= ns) m2[i] = -INFINITY;
      }
    }
    float M = -INFINITY;
    if constexpr (!BATCHED) {
      int s = 0;
      for (; s + 4 <= ns; s += 4) {  // four loads per wait
        float mb[4];
#pragma unroll
        for (int i = 0; i < 4; i++) mb[i] = m[((size_t)(s + i) * n_sets + set) * 16 + r];
        M = fmaxf(M, fmaxf(fmaxf(mb[0], mb[1]), fmaxf(mb[2], mb[3])));
      }
      for (; s < ns; s++) M = fmaxf(M, m[((size_t)s * n_sets + set) * 16 + r]);
    } else {
      for (int s = 0; s < ns; s += kBatch) {
        float mb[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; i++)
          mb[i] = s + i < ns ? m[((size_t)(s + i) * n_sets + set) * 16 + r] : -INFINITY;
#pragma unroll
        for (int i = 0; i < kBatch; i++) M = fmaxf(M, mb[i]);
      }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    double lacc = 0.0;
    if (M != -INFINITY && !BATCHED) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        if (m2[i] == -INFINITY) continue;
        acc += fast_exp2(m2[i] - M) * o2[i];
        if (c == 0) lacc += exp2((double)m2[i] - (double)M) * l2[i];
      }
    } else if (M != -INFINITY) {  // a split past the end reads split s, weighted 0
#pragma unroll
      for (int i = 0; i < kBatch; i++) {
        if (mb0[i] == -INFINITY) continue;
        acc += fast_exp2(mb0[i] - M) * ob0[i];
        if (c == 0) lacc += exp2((double)mb0[i] - (double)M) * lb0[i];
      }
      for (int s = sl + kBatch * SP; s < ns; s += kBatch * SP) {
        float mb[kBatch];
        f32x4 ob[kBatch];
        double lb[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; i++) {
          const int si = s + i * SP;
          const size_t prow = ((size_t)(si < ns ? si : s) * n_sets + set) * 16 + r;
          mb[i] = si < ns ? m[prow] : -INFINITY;
          ob[i] = *(const f32x4*)(p.po[br] + prow * D + 4 * c);
          lb[i] = c == 0 ? p.l[br][prow] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < kBatch; i++) {
          if (mb[i] == -INFINITY) continue;
          acc += fast_exp2(mb[i] - M) * ob[i];
          if (c == 0) lacc += exp2((double)mb[i] - (double)M) * lb[i];
        }
      }
    }
    *(f32x4*)&red[sl][4 * c] = acc;
    if (c == 0) redl[sl] = lacc;
    __syncthreads();
    if (sl == 0) {
      double L = 0.0;
      for (int q = 0; q < SP; q++) L += redl[q];
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < SP; q++)
#pragma unroll
        for (int e = 0; e < 4; e++) sum[e] += red[q][4 * c + e];
      double wgt = og;
      if (p.n_branch == 2 && !p.gate_ch) {
        const float z = p.gate[orow * 2 + br];
        wgt *= 1.0 / (1.0 + exp(-(double)z));
      }
      const RowNorm n = row_norm(M, L, p.sink[br], hr, wgt);
      if (p.gate_ch) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float gb = p.n_branch == 2 ? sigmoid_f(p.gate[(orow * 2 + br) * D + 4 * c + e])
                                           : 1.f;
          out[e] += sum[e] * n.factor * gb * og_ch[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) out[e] += sum[e] * n.factor;
      }
      if (br == 0 && c == 0) lse0 = n.lse;
    }
    __syncthreads();
  }
  if (sl != 0) return;
  const size_t ooff = (((size_t)b * p.Tq + jr) * p.Hq + hr) * D + 4 * c;
  if (p.out_f32) {
#pragma unroll
    for (int e = 0; e < 4; e++) ((float*)p.o)[ooff + e] = out[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; e++) ((uint16_t*)p.o)[ooff + e] = f2bf(out[e]);
  }
  if (p.lse && c == 0) p.lse[((size_t)b * p.Hq + hr) * p.Tq + jr] = (float)lse0;
}

// Workgroups of a row-kernel launch: one per (row-set, split).
unsigned ra_grid(const RowAttnParams& p) {
  return (unsigned)((long long)p.B * p.Hkv * p.sets_per_bu * p.cpq * p.n_split);
}

template <int D, bool F32, int NW>
hipError_t launch_ra_paged(const RowAttnParams& p, KeySrc src, bool gated, hipStream_t stream) {
  const dim3 grid(ra_grid(p));
  const int threads = 64 * NW;
  if (gated) {
    if constexpr (D > 128) {
      return hipErrorInvalidValue;  // registers: one branch per launch
    } else {
      if (src == SRC_TOKEN)
        row_attn_kernel<D, F32, SRC_TOKEN, true, NW, false, true><<<grid, threads, 0, stream>>>(p);
      else if (src == SRC_BLOCK)
        row_attn_kernel<D, F32, SRC_BLOCK, true, NW, false, true><<<grid, threads, 0, stream>>>(p);
      else
        return hipErrorInvalidValue;
      return hipGetLastError();
    }
  }
  switch (src) {
    case SRC_RANGE:
      if constexpr (NW == 4) {
        if (p.logits)
          row_attn_kernel<D, F32, SRC_RANGE, false, 4, true, true><<<grid, threads, 0, stream>>>(p);
        else
          row_attn_kernel<D, F32, SRC_RANGE, false, 4, false, true><<<grid, threads, 0, stream>>>(p);
        break;
      }
      return hipErrorInvalidValue;
    case SRC_TOKEN: row_attn_kernel<D, F32, SRC_TOKEN, false, NW, false, true><<<grid, threads, 0, stream>>>(p); break;
    case SRC_BLOCK: row_attn_kernel<D, F32, SRC_BLOCK, false, NW, false, true><<<grid, threads, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;  // the window source is never paged
  }
  return hipGetLastError();
}

template <int D, bool F32, int NW>
hipError_t launch_ra(const RowAttnParams& p, KeySrc src, bool gated, hipStream_t stream) {
  if (p.pages) return launch_ra_paged<D, F32, NW>(p, src, gated, stream);
  const dim3 grid(ra_grid(p));
  const int threads = 64 * NW;
  if (p.logits) {
    if constexpr (NW == 4) {
      if (src != SRC_RANGE || gated) return hipErrorInvalidValue;
      row_attn_kernel<D, F32, SRC_RANGE, false, 4, true><<<grid, threads, 0, stream>>>(p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (gated) {
    if constexpr (D > 128) {
      return hipErrorInvalidValue;  // registers: one branch per launch
    } else {
      if (src == SRC_TOKEN)
        row_attn_kernel<D, F32, SRC_TOKEN, true, NW><<<grid, threads, 0, stream>>>(p);
      else
        row_attn_kernel<D, F32, SRC_BLOCK, true, NW><<<grid, threads, 0, stream>>>(p);
      return hipGetLastError();
    }
  }
  switch (src) {
    case SRC_RANGE: row_attn_kernel<D, F32, SRC_RANGE, false, NW><<<grid, threads, 0, stream>>>(p); break;
    case SRC_TOKEN: row_attn_kernel<D, F32, SRC_TOKEN, false, NW><<<grid, threads, 0, stream>>>(p); break;
    case SRC_BLOCK: row_attn_kernel<D, F32, SRC_BLOCK, false, NW><<<grid, threads, 0, stream>>>(p); break;
    case SRC_WINDOW: row_attn_kernel<D, F32, SRC_WINDOW, false, NW><<<grid, threads, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

template <int D, bool F32, bool PAGED>
hipError_t launch_two(const RowAttnParams& pg, const RowAttnParams& pl, KeySrc src,
                      hipStream_t stream) {
  const int n_glob = (int)ra_grid(pg);
  const dim3 grid(n_glob + ra_grid(pl));
  if (src == SRC_TOKEN)
    row_attn_two_kernel<D, F32, SRC_TOKEN, 4, PAGED><<<grid, 256, 0, stream>>>(pg, pl, n_glob);
  else if (src == SRC_BLOCK)
    row_attn_two_kernel<D, F32, SRC_BLOCK, 4, PAGED><<<grid, 256, 0, stream>>>(pg, pl, n_glob);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_two_d(const RowAttnParams& pg, const RowAttnParams& pl, KeySrc src,
                        hipStream_t stream) {
  return pg.pages ? launch_two<D, F32, true>(pg, pl, src, stream)
                  : launch_two<D, F32, false>(pg, pl, src, stream);
}

}  // namespace

hipError_t launch_row_attn_two(const RowAttnParams& pg, const RowAttnParams& pl, int head_dim,
                               bool in_f32, KeySrc src, hipStream_t stream) {
  if (pg.final_direct || pl.final_direct || pl.pages) return hipErrorInvalidValue;
  if (head_dim == 256) {
    if (in_f32) return hipErrorInvalidValue;
    return launch_two_d<256, false>(pg, pl, src, stream);
  }
  if (head_dim == 128)
    return in_f32 ? launch_two_d<128, true>(pg, pl, src, stream)
                  : launch_two_d<128, false>(pg, pl, src, stream);
  return in_f32 ? launch_two_d<64, true>(pg, pl, src, stream)
                : launch_two_d<64, false>(pg, pl, src, stream);
}

hipError_t launch_row_attn(const RowAttnParams& p, int head_dim, bool in_f32, KeySrc src,
                           hipStream_t stream, bool gated, bool wide) {
  if (wide) {  // 8 waves: bf16 only (the fp32 variants need more registers than that allows)
    if (in_f32) return hipErrorInvalidValue;
    return head_dim == 128 ? launch_ra<128, false, 8>(p, src, gated, stream)
                           : launch_ra<64, false, 8>(p, src, gated, stream);
  }
  if (head_dim == 256) {  // bf16, 4 waves, one branch per launch (registers allow no more)
    if (in_f32 || gated) return hipErrorInvalidValue;
    return launch_ra<256, false, 4>(p, src, false, stream);
  }
  if (head_dim == 128)
    return in_f32 ? launch_ra<128, true, 4>(p, src, gated, stream)
                  : launch_ra<128, false, 4>(p, src, gated, stream);
  return in_f32 ? launch_ra<64, true, 4>(p, src, gated, stream)
                : launch_ra<64, false, 4>(p, src, gated, stream);
}

template <int D>
void launch_combine_d(const CombineParams& p, dim3 grid, hipStream_t stream) {
  constexpr int SP = 256 / (D / 4);  // split lanes of the kernel
  int most = p.n_split[0];
  if (p.n_branch == 2 && p.n_split[1] > most) most = p.n_split[1];
  if (most > 2 * SP)
    combine_kernel<D, true><<<grid, 256, 0, stream>>>(p);
  else
    combine_kernel<D, false><<<grid, 256, 0, stream>>>(p);
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  // one workgroup per row of every row-set (a last, partial query chunk leaves some idle)
  const dim3 grid(p.B * p.Hkv * p.sets_per_bu * p.cpq * p.q_per_set * p.hpc);
  if (head_dim == 256)
    launch_combine_d<256>(p, grid, stream);
  else if (head_dim == 128)
    launch_combine_d<128>(p, grid, stream);
  else
    launch_combine_d<64>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace hs
