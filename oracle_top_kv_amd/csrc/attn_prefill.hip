// attn_prefill.hip -- full causal GQA attention for many queries per KV head (prefill):
// O and LSE [P2 "Extracting block scores from exact attention", attention equations;
// P4 section 3.2, the tiled loop of Algorithm 1 without its score output].
//
// A workgroup owns 256 (query, head) rows of one KV head: 256/g consecutive queries times the
// g heads of the group, so every K/V tile staged in LDS serves all heads of the group (256 rows
// per 64-key tile: 128 flop per byte of K/V moved from L2).  Each of the 8 waves owns 32 rows
// (two 16-row MFMA blocks).  Per 64-key tile:
//   S^T = K Q^T   A = K from LDS (ds_read_b128), B = Q^T resident in registers
//   online softmax in the log2 domain; the row state lives in the 4 lanes of the row
//   O^T += V^T P^T  B = P^T straight from the S^T accumulator (bf16), A = V^T from the
//                   row-major LDS tile with ds_read_b64_tr_b16
// K/V tiles are double-buffered: the next tile's rows are loaded into registers while the
// current tile is computed, then stored to the other buffer; one barrier per tile.  Only tiles
// that reach past the earliest query position of the workgroup apply the causal mask.
#include "hs_device.h"
#include "hs_kernels.h"

namespace hs {
namespace {

constexpr int kRowsWG = 256;
constexpr int kThreads = 512;
constexpr int kBN = 64;

template <int D>
struct PfCfg {
  static constexpr int KStr = D + 8;    // K tile row stride (elements): conflict-free ds_read_b128
  static constexpr int VStr = D + 16;   // V tile row stride: conflict-free transpose reads
  static constexpr int KK = D / 32;     // MFMA steps over d
  static constexpr int DB = D / 16;     // 16-wide d blocks of O
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int LPT = kBN * CPR / kThreads;  // chunks per thread per tile (each of K and V)
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void pf_attn_kernel(PrefillParams p) {
  using C = PfCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kBN * C::KStr];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][kBN * C::VStr];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rn = lane & 15, jg = lane >> 4;
  const int qpw = kRowsWG / p.g;  // queries per workgroup
  const int n_qt = (p.Tq + qpw - 1) / qpw;
  // KV head fastest, then query tile (latest, i.e. longest, first), then batch
  const int u = blockIdx.x % p.Hkv;
  const int qt = n_qt - 1 - (int)((blockIdx.x / p.Hkv) % n_qt);
  const int b = blockIdx.x / (p.Hkv * n_qt);
  const int j0 = qt * qpw;
  const int nq = min(qpw, p.Tq - j0);
  const long long t_min = p.q_off + j0;
  const long long t_max = p.q_off + j0 + nq - 1;

  // this lane's two rows (one per 16-row block)
  bool row_ok[2];
  long long t_row[2];
  int j_row[2], h_row[2];
  bf16x8 qb[2][C::KK];
#pragma unroll
  for (int rb = 0; rb < 2; rb++) {
    const int r = wave * 32 + rb * 16 + rn;
    const int jq = r / p.g, hh = r % p.g;
    row_ok[rb] = jq < nq;
    j_row[rb] = j0 + (row_ok[rb] ? jq : 0);
    h_row[rb] = u * p.g + hh;
    t_row[rb] = p.q_off + j_row[rb];
    const uint16_t* qp = (const uint16_t*)p.q + (((size_t)b * p.Tq + j_row[rb]) * p.Hq + h_row[rb]) * D;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++) {
      u32x4 raw = row_ok[rb] ? *(const u32x4*)(qp + 32 * kk + 8 * jg) : u32x4{0, 0, 0, 0};
      qb[rb][kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_s[2] = {0.f, 0.f}, l_c[2] = {0.f, 0.f};
  f32x4 oacc[2][C::DB];
#pragma unroll
  for (int rb = 0; rb < 2; rb++)
#pragma unroll
    for (int db = 0; db < C::DB; db++) oacc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t kv_row_stride = (size_t)p.Hkv * D;
  const uint16_t* kbase = (const uint16_t*)p.k + ((size_t)b * p.Tk * p.Hkv + u) * D;
  const uint16_t* vbase = (const uint16_t*)p.v + ((size_t)b * p.Tk * p.Hkv + u) * D;
  const int n_tiles = (int)((t_max + kBN) / kBN);  // tiles covering keys 0..t_max

  u32x4 kreg[C::LPT], vreg[C::LPT];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::LPT; i++) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / C::CPR, ch = c % C::CPR;
      long long key = (long long)t * kBN + row;
      if (key > t_max) key = t_max;  // rows past the last query are loaded but masked
      kreg[i] = *(const u32x4*)(kbase + (size_t)key * kv_row_stride + ch * 8);
      vreg[i] = ld_stream(vbase + (size_t)key * kv_row_stride + ch * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LPT; i++) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / C::CPR, ch = c % C::CPR;
      *(u32x4*)(&ks[buf][row * C::KStr + ch * 8]) = kreg[i];
      *(u32x4*)(&vs[buf][row * C::VStr + ch * 8]) = vreg[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; t++) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const long long key0 = (long long)t * kBN;
    const bool need_mask = key0 + kBN - 1 > t_min;

    // S^T for 4 key blocks x 2 row blocks
    f32x4 sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      sacc[kb][0] = sacc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KK; kk++) {
        const bf16x8 ka = *(const bf16x8*)(&ks[buf][(16 * kb + rn) * C::KStr + 32 * kk + 8 * jg]);
        sacc[kb][0] = mfma_bf16(ka, qb[0][kk], sacc[kb][0]);
        sacc[kb][1] = mfma_bf16(ka, qb[1][kk], sacc[kb][1]);
      }
    }

    bf16x8 pb[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
      float sv[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          float x = sacc[kb][rb][e] * p.scale_log2;
          if (need_mask) {
            const long long key = key0 + 16 * kb + 4 * jg + e;
            if (!row_ok[rb] || key > t_row[rb]) x = -INFINITY;
          }
          sv[kb][e] = x;
          mx = fmaxf(mx, x);
        }
      mx = max4groups(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[rb] - m_use);
      float pv[4][4];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          pv[kb][e] = fast_exp2(sv[kb][e] - m_use);
          psum += pv[kb][e];
        }
      l_s[rb] *= alpha;
      l_c[rb] *= alpha;
      kahan_add(l_s[rb], l_c[rb], psum);
      m_run[rb] = m_new;
      if (__ballot(alpha != 1.f)) {  // rescale only when some row maximum moved
#pragma unroll
        for (int db = 0; db < C::DB; db++) oacc[rb][db] *= alpha;
      }
#pragma unroll
      for (int s = 0; s < 2; s++) {
        const float x8[8] = {pv[2 * s][0], pv[2 * s][1], pv[2 * s][2], pv[2 * s][3],
                             pv[2 * s + 1][0], pv[2 * s + 1][1], pv[2 * s + 1][2], pv[2 * s + 1][3]};
        pb[rb][s] = pack_bf16x8(x8);
      }
    }

    // O^T += V^T P^T over the two 32-key halves of the tile
#pragma unroll
    for (int s = 0; s < 2; s++) {
#pragma unroll
      for (int db = 0; db < C::DB; db++) {
        const uint16_t* a0 = &vs[buf][(32 * s + 4 * jg + (rn >> 2)) * C::VStr + 16 * db + 4 * (rn & 3)];
        const bf16x8 va = join_tr(lds_read_tr16(a0), lds_read_tr16(a0 + 16 * C::VStr));
        oacc[0][db] = mfma_bf16(va, pb[0][s], oacc[0][db]);
        oacc[1][db] = mfma_bf16(va, pb[1][s], oacc[1][db]);
      }
    }
    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: normalize and write O and LSE
#pragma unroll
  for (int rb = 0; rb < 2; rb++) {
    double ld = (double)l_s[rb] - (double)l_c[rb];
    ld += __shfl_xor(ld, 16, 64);
    ld += __shfl_xor(ld, 32, 64);
    if (!row_ok[rb]) continue;
    const float inv = ld > 0.0 ? (float)(1.0 / ld) : 0.f;
    const size_t ooff = (((size_t)b * p.Tq + j_row[rb]) * p.Hq + h_row[rb]) * D + 4 * jg;
#pragma unroll
    for (int db = 0; db < C::DB; db++) {
      const f32x4 o4 = oacc[rb][db] * inv;
      if (p.out_f32) {
        *(f32x4*)((float*)p.o + ooff + 16 * db) = o4;
      } else {
        typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
        u16x4 h4 = {f2bf(o4[0]), f2bf(o4[1]), f2bf(o4[2]), f2bf(o4[3])};
        *(u16x4*)((uint16_t*)p.o + ooff + 16 * db) = h4;
      }
    }
    if (jg == 0)
      p.lse[((size_t)b * p.Hq + h_row[rb]) * p.Tq + j_row[rb]] =
          ld > 0.0 ? (float)(((double)m_run[rb] + log2(ld)) * kLn2) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_attn(const PrefillParams& p, int head_dim, hipStream_t stream) {
  const int qpw = kRowsWG / p.g;
  const int n_qt = (p.Tq + qpw - 1) / qpw;
  const dim3 grid(p.B * p.Hkv * n_qt);
  if (head_dim == 128)
    pf_attn_kernel<128><<<grid, kThreads, 0, stream>>>(p);
  else
    pf_attn_kernel<64><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace hs
