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
#include "hs_device.h"
#include "hs_kernels.h"

namespace hs {
namespace {

constexpr int kWaves = 4;
constexpr int kStep = 32;  // keys per wave step

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, bool F32>
struct RaCfg {
  static constexpr int kElem = F32 ? 4 : 2;
  static constexpr int kVStride = D + (F32 ? 4 : 16);  // LDS row stride (elements), padded
  static constexpr int kChunksPerRow = D * kElem / 16;
  static constexpr int kVLoads = kStep * kChunksPerRow / 64;  // 16-byte V chunks per lane
  static constexpr int kVTileBytes = kStep * kVStride * kElem;
  static constexpr int kCombineBytes = kWaves * 16 * D * 4 + kWaves * 16 * 4 + kWaves * 16 * 8;
  static constexpr int kSmem =
      (kWaves * kVTileBytes > kCombineBytes ? kWaves * kVTileBytes : kCombineBytes);
};

template <int SRC>
__device__ __forceinline__ int entry_pos(const RowAttnParams& p, int e, int L, long long lo,
                                         long long t_last, const int32_t* list) {
  if (e >= L) return -1;
  if (SRC == SRC_RANGE) return (int)(lo + e);
  if (SRC == SRC_TOKEN) {
    const int x = list[e];
    return (x >= 0 && x <= t_last) ? x : -1;
  }
  const int blk = list[e / p.block];
  if (blk < 0 || (long long)blk > t_last / p.block) return -1;
  const long long x = (long long)blk * p.block + e % p.block;
  return x <= t_last ? (int)x : -1;
}

template <int D, bool F32, int SRC>
__global__ __launch_bounds__(256) void row_attn_kernel(RowAttnParams p) {
  using Cfg = RaCfg<D, F32>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::kSmem];
  __shared__ int pos_lds[kWaves][kStep];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rn = lane & 15;   // MFMA row / column index of this lane
  const int jg = lane >> 4;   // lane group 0..3
  const int split = blockIdx.x;
  const int set = blockIdx.y;
  const int sq = set % p.sets_per_bu;
  const int bu = set / p.sets_per_bu;
  const int u = bu % p.Hkv;
  const int b = bu / p.Hkv;
  const int j0 = sq * p.q_per_set;
  const int nq = min(p.q_per_set, p.Tq - j0);
  const int nrows = nq * p.g;
  const long long t_first = p.q_off + j0;
  const long long t_last = p.q_off + j0 + nq - 1;

  int L;
  long long lo = 0;
  const int32_t* list = nullptr;
  if (SRC == SRC_RANGE) {
    lo = (p.window > 0) ? (t_first - p.window + 1 > 0 ? t_first - p.window + 1 : 0) : 0;
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
  const int jq = row_ok ? rn / p.g : 0;
  const int hh = row_ok ? rn % p.g : 0;
  const long long t_row = p.q_off + j0 + jq;
  const int h = u * p.g + hh;
  const long long lo_row = (SRC == SRC_RANGE && p.window > 0) ? t_row - p.window + 1 : 0;

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
  const int step_begin = split * p.steps_per_split;
  const int step_end = min(step_begin + p.steps_per_split, n_steps);
  unsigned char* vtile = smem + wave * Cfg::kVTileBytes;
  int* pos_w = pos_lds[wave];

  for (int step = step_begin + wave; step < step_end; step += kWaves) {
    if (lane < kStep) pos_w[lane] = entry_pos<SRC>(p, step * kStep + lane, L, lo, t_last, list);
    wave_lds_sync();

    // K operand for the two 16-key blocks (straight from HBM)
    const int pk0 = pos_w[rn], pk1 = pos_w[16 + rn];
    f32x4 sacc[2];
    if constexpr (!F32) {
      const uint16_t* kp0 = (const uint16_t*)p.k + kv_base + (size_t)(pk0 < 0 ? 0 : pk0) * kv_row_stride;
      const uint16_t* kp1 = (const uint16_t*)p.k + kv_base + (size_t)(pk1 < 0 ? 0 : pk1) * kv_row_stride;
      u32x4 ka0[KK], ka1[KK];
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        ka0[kk] = *(const u32x4*)(kp0 + 32 * kk + 8 * jg);
        ka1[kk] = *(const u32x4*)(kp1 + 32 * kk + 8 * jg);
      }
      // V rows -> LDS tile (row-major [key][d], padded rows)
#pragma unroll
      for (int n = 0; n < Cfg::kVLoads; n++) {
        const int c = n * 64 + lane;
        const int e = c / Cfg::kChunksPerRow, qc = c % Cfg::kChunksPerRow;
        const int pv = pos_w[e];
        const uint16_t* vp = (const uint16_t*)p.v + kv_base + (size_t)(pv < 0 ? 0 : pv) * kv_row_stride + qc * 8;
        *(u32x4*)((uint16_t*)vtile + e * Cfg::kVStride + qc * 8) = *(const u32x4*)vp;
      }
      sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        sacc[0] = mfma_bf16(__builtin_bit_cast(bf16x8, ka0[kk]), qb[kk], sacc[0]);
        sacc[1] = mfma_bf16(__builtin_bit_cast(bf16x8, ka1[kk]), qb[kk], sacc[1]);
      }
    } else {
      const float* kp0 = (const float*)p.k + kv_base + (size_t)(pk0 < 0 ? 0 : pk0) * kv_row_stride + jg * KK;
      const float* kp1 = (const float*)p.k + kv_base + (size_t)(pk1 < 0 ? 0 : pk1) * kv_row_stride + jg * KK;
      float ka0[KK], ka1[KK];
#pragma unroll
      for (int s = 0; s < KK; s++) {
        ka0[s] = kp0[s];
        ka1[s] = kp1[s];
      }
#pragma unroll
      for (int n = 0; n < Cfg::kVLoads; n++) {
        const int c = n * 64 + lane;
        const int e = c / Cfg::kChunksPerRow, qc = c % Cfg::kChunksPerRow;
        const int pv = pos_w[e];
        const float* vp = (const float*)p.v + kv_base + (size_t)(pv < 0 ? 0 : pv) * kv_row_stride + qc * 4;
        *(u32x4*)((float*)vtile + e * Cfg::kVStride + qc * 4) = *(const u32x4*)vp;
      }
      sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KK; s++) {
        sacc[0] = mfma_f32(ka0[s], qf[s], sacc[0]);
        sacc[1] = mfma_f32(ka1[s], qf[s], sacc[1]);
      }
    }

    // scale to the log2 domain and mask
    float sv[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int pos = pos_w[16 * kb + 4 * jg + e];
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
        const bf16x8 va = join_tr(lds_read_tr16(a0), lds_read_tr16(a1));
        oacc[db] = mfma_bf16(va, pb, oacc[db]);
      }
    } else {
      const float* vt = (const float*)vtile;
#pragma unroll
      for (int db = 0; db < D / 16; db++)
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float va = vt[(16 * kb + 4 * jg + e) * Cfg::kVStride + 16 * db + rn];
            oacc[db] = mfma_f32(va, pv8[4 * kb + e], oacc[db]);
          }
    }
    wave_lds_sync();  // tile reads done before the next step overwrites it
  }

  // ---- merge the 4 waves of this workgroup ----
  __syncthreads();
  float* cO = (float*)smem;                     // [kWaves][16][D]
  float* cM = cO + kWaves * 16 * D;             // [kWaves][16]
  double* cL = (double*)(cM + kWaves * 16);     // [kWaves][16]
#pragma unroll
  for (int db = 0; db < D / 16; db++)
#pragma unroll
    for (int e = 0; e < 4; e++) cO[(wave * 16 + rn) * D + 16 * db + 4 * jg + e] = oacc[db][e];
  double ld = (double)l_s - (double)l_c;
  ld += __shfl_xor(ld, 16, 64);
  ld += __shfl_xor(ld, 32, 64);
  if (jg == 0) {
    cM[wave * 16 + rn] = m_run;
    cL[wave * 16 + rn] = ld;
  }
  __syncthreads();

  constexpr int CPT = D / 16;  // columns per thread
  const int r = threadIdx.x >> 4;
  const int c0 = (threadIdx.x & 15) * CPT;
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
  float ov[CPT];
#pragma unroll
  for (int c = 0; c < CPT; c++) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) acc += f[w] * cO[(w * 16 + r) * D + c0 + c];
    ov[c] = acc;
  }
  if (r >= nrows) return;
  const int jr = j0 + r / p.g;
  const int hr = u * p.g + r % p.g;
  if (p.final_direct) {
    const float inv = (Ls > 0.0) ? (float)(1.0 / Ls) : 0.f;
    const size_t ooff = (((size_t)b * p.Tq + jr) * p.Hq + hr) * D + c0;
    if (p.out_f32) {
      float* op = (float*)p.o + ooff;
#pragma unroll
      for (int c = 0; c < CPT; c++) op[c] = ov[c] * inv;
    } else {
      uint16_t* op = (uint16_t*)p.o + ooff;
#pragma unroll
      for (int c = 0; c < CPT; c++) op[c] = f2bf(ov[c] * inv);
    }
    if (p.lse && c0 == 0)
      p.lse[((size_t)b * p.Hq + hr) * p.Tq + jr] =
          (Ls > 0.0) ? (float)(((double)M + log2(Ls)) * kLn2) : -INFINITY;
  } else {
    const size_t n_sets = gridDim.y;
    const size_t prow = ((size_t)split * n_sets + set) * 16 + r;
    if (c0 == 0) {
      p.part_m[prow] = M;
      p.part_l[prow] = Ls;
    }
#pragma unroll
    for (int c = 0; c < CPT; c++) p.part_o[prow * D + c0 + c] = ov[c];
  }
}

// ---- split / branch combine ---------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int CPT = D / 16;
  const int set = blockIdx.x;
  const size_t n_sets = gridDim.x;
  const int r = threadIdx.x >> 4;
  const int c0 = (threadIdx.x & 15) * CPT;
  const int sq = set % p.sets_per_bu;
  const int bu = set / p.sets_per_bu;
  const int u = bu % p.Hkv;
  const int b = bu / p.Hkv;
  const int j0 = sq * p.q_per_set;
  const int nq = min(p.q_per_set, p.Tq - j0);
  if (r >= nq * p.g) return;
  const int jr = j0 + r / p.g;
  const int hr = u * p.g + r % p.g;

  double out[CPT];
  double lse0 = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPT; c++) out[c] = 0.0;
  for (int br = 0; br < p.n_branch; br++) {
    float M = -INFINITY;
    for (int s = 0; s < p.n_split[br]; s++) M = fmaxf(M, p.m[br][((size_t)s * n_sets + set) * 16 + r]);
    double Ls = 0.0, acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; c++) acc[c] = 0.0;
    if (M != -INFINITY) {
      for (int s = 0; s < p.n_split[br]; s++) {
        const size_t prow = ((size_t)s * n_sets + set) * 16 + r;
        const float ms = p.m[br][prow];
        if (ms == -INFINITY) continue;
        const double f = exp2((double)ms - (double)M);
        Ls += f * p.l[br][prow];
#pragma unroll
        for (int c = 0; c < CPT; c++) acc[c] += f * (double)p.po[br][prow * D + c0 + c];
      }
    }
    double wgt = 1.0;
    if (p.n_branch == 2) {
      const float z = p.gate[(((size_t)b * p.Tq + jr) * p.Hq + hr) * 2 + br];
      wgt = 1.0 / (1.0 + exp(-(double)z));
    }
    const double inv = Ls > 0.0 ? wgt / Ls : 0.0;
#pragma unroll
    for (int c = 0; c < CPT; c++) out[c] += acc[c] * inv;
    if (br == 0) lse0 = Ls > 0.0 ? ((double)M + log2(Ls)) * kLn2 : -INFINITY;
  }
  const size_t ooff = (((size_t)b * p.Tq + jr) * p.Hq + hr) * D + c0;
  if (p.out_f32) {
#pragma unroll
    for (int c = 0; c < CPT; c++) ((float*)p.o)[ooff + c] = (float)out[c];
  } else {
#pragma unroll
    for (int c = 0; c < CPT; c++) ((uint16_t*)p.o)[ooff + c] = f2bf((float)out[c]);
  }
  if (p.lse && c0 == 0) p.lse[((size_t)b * p.Hq + hr) * p.Tq + jr] = (float)lse0;
}

template <int D, bool F32>
hipError_t launch_ra(const RowAttnParams& p, KeySrc src, hipStream_t stream) {
  const dim3 grid(p.n_split, p.B * p.Hkv * p.sets_per_bu);
  switch (src) {
    case SRC_RANGE: row_attn_kernel<D, F32, SRC_RANGE><<<grid, 256, 0, stream>>>(p); break;
    case SRC_TOKEN: row_attn_kernel<D, F32, SRC_TOKEN><<<grid, 256, 0, stream>>>(p); break;
    case SRC_BLOCK: row_attn_kernel<D, F32, SRC_BLOCK><<<grid, 256, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_row_attn(const RowAttnParams& p, int head_dim, bool in_f32, KeySrc src,
                           hipStream_t stream) {
  if (head_dim == 128) return in_f32 ? launch_ra<128, true>(p, src, stream) : launch_ra<128, false>(p, src, stream);
  return in_f32 ? launch_ra<64, true>(p, src, stream) : launch_ra<64, false>(p, src, stream);
}

hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(p.B * p.Hkv * p.sets_per_bu);
  if (head_dim == 128)
    combine_kernel<128><<<grid, 256, 0, stream>>>(p);
  else
    combine_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace hs
