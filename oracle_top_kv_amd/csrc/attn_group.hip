// attn_group.hip -- full attention of one query over a long key range for GQA groups of 32, 48
// or 64 query heads per KV head (decode in HySparse2's head shape: 64 query heads on one KV
// head, d = 256) [P2 "Extracting block scores from exact attention": a = q.k/sqrt(d),
// p = softmax, o = sum p v; P1 section 4.2 and P5 model configuration for the head shape].
//
// One workgroup per (batch entry, KV head, query, key split) with one wave per 16-head chunk of
// the group (two over a contiguous key range at d 256, each taking half of every step's keys).  Every 64-key step of K and V is loaded once by the whole workgroup into LDS
// (double-buffered, through buffer loads whose descriptors hold the step's first row and its
// number of rows) and read there by every chunk: K and V cross HBM and L2 once, however many
// heads share them.  Per wave the arithmetic is the row kernel's:
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 d from the LDS tile, B = Q^T
//                  resident; lane (row n, group j) holds S[n][16kb + 4j .. 16kb + 4j + 3]
//   online softmax in the log2 domain, Kahan-compensated row sums in the 4 lanes of a row
//   O^T += V^T P^T B = P^T straight from the S^T accumulator, A = V^T read from the row-major
//                  V tile with ds_read_b64_tr_b16 (keys in the accumulator's order)
// Key sources: the contiguous range 0..t (full attention), or a token / block index list of
// (b, t, u) (the sparse layers' global branch [P2 "Cross-layer KV cache reuse"; P2 "Same query,
// two memories"]): a split's list positions are staged in LDS first, and each step gathers its
// 64 rows straight into the shared tile (invalid entries read as zeros and are masked).
// LOGITS (range only): the raw dot products q.k go to a [B, Tq, Hq, Tk] array, 16 bytes per
// lane per key block (64 contiguous bytes per row).  With several splits every workgroup writes
// split partials (row maximum, row sum, unnormalized O) and the combine kernel normalizes; with
// one split (final_direct) the workgroup normalizes its rows itself (sink, output gate) and
// writes O and the LSE.
#include "hs_device.h"
#include "hs_kernels.h"

namespace hs {
namespace {

constexpr int kGStep = 64;                   // keys per step
constexpr int kBufferConfig = 0x00020000;    // buffer descriptor word 3 (gfx9 family: raw dwords)
constexpr int kNonTemporal = 2;              // cache-policy bit of a buffer load: non-temporal

template <int D>
struct GaCfg {
  static constexpr int KStr = D + 8;   // K tile row stride (elements): conflict-free b128 reads
  static constexpr int VStr = D + 16;  // V tile row stride: conflict-free transpose reads
  static constexpr int KK = D / 32;    // MFMA steps over d
  static constexpr int DB = D / 16;    // 16-wide d blocks of O^T
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int kChunks = kGStep * CPR;  // 16-byte chunks per tile
};

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kMaxSplitEntries = 2048;  // list entries staged per workgroup (32 steps)

// Waves per 16-head chunk: over a contiguous key range at d 256, each chunk of a group of 32 or
// 64 heads has two waves, one per 32-key half of every step (two waves per SIMD at 64 heads, so
// that one covers the other's LDS and MFMA latencies; registers allow no more, and with 48 heads
// six waves would spill); the halves are merged at the end.  Index lists keep one wave per
// chunk: their splits are one or two steps long, too short to repay the merge.
template <int D, int NW, int SRC>
constexpr int key_halves() {
  return D == 256 && NW % 2 == 0 && SRC == SRC_RANGE ? 2 : 1;
}

template <int D, int NW, int SRC, bool LOGITS>
__global__ __launch_bounds__((64 * NW * key_halves<D, NW, SRC>()), 1) void group_attn_kernel(RowAttnParams p) {
  using C = GaCfg<D>;
  static_assert(!LOGITS || SRC == SRC_RANGE, "logits come from the full-attention pass only");
  constexpr bool kList = SRC == SRC_TOKEN || SRC == SRC_BLOCK;
  constexpr int KH = key_halves<D, NW, SRC>();
  constexpr int kKeys = kGStep / KH;  // keys of a step per wave
  constexpr int kKB = kKeys / 16;     // 16-key blocks per wave and step
  constexpr int kThreads = 64 * NW * KH;
  constexpr int kPer = (C::kChunks + kThreads - 1) / kThreads;  // chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][kGStep * C::KStr];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kGStep * C::VStr];
  __shared__ int pos_all[kList ? kMaxSplitEntries : 1];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hc = wave % NW, kh = wave / NW;  // head chunk, key half
  const int rn = lane & 15, jg = lane >> 4;
  // KV head fastest, then split, then (batch, query)
  const int x = blockIdx.x;
  const int u = x % p.Hkv;
  const int split = (x / p.Hkv) % p.n_split;
  const int bq = x / (p.Hkv * p.n_split);
  const int j = bq % p.Tq;
  const int b = bq / p.Tq;
  const long long t_row = p.q_off + j;  // this query's position: keys 0 .. t_row
  // the last chunk of a group that is not a multiple of 16 heads has rows without a head
  const bool row_ok = hc * 16 + rn < p.g;
  const int h = u * p.g + hc * 16 + (row_ok ? rn : 0);

  // list modes: the (b, t, u) list and its number of keys L (blocks count block keys each)
  const int32_t* list = nullptr;
  int L = (int)(t_row + 1);
  if constexpr (kList) {
    const size_t lrow = ((size_t)b * p.Tq + j) * p.Hkv + u;
    list = p.idx + lrow * p.idx_cap;
    int c = p.cnt[lrow];
    c = c < 0 ? 0 : (c > p.idx_cap ? p.idx_cap : c);
    L = SRC == SRC_TOKEN ? c : c * p.block;
  }
  const int n_steps = (L + kGStep - 1) / kGStep;
  const int s0 = split * p.steps_per_split;
  const int s1 = min(s0 + p.steps_per_split, n_steps);
  // position of list entry e (-1: none, past the count, or after t), as in the row kernel
  auto entry_pos = [&](int e) -> int {
    if (e >= L) return -1;
    if constexpr (SRC == SRC_TOKEN) {
      const int x = list[e];
      return (x >= 0 && x <= t_row) ? x : -1;
    } else {
      const int blk = list[e / p.block];
      if (blk < 0 || (long long)blk > t_row / p.block) return -1;
      const long long x = (long long)blk * p.block + e % p.block;
      return x <= t_row ? (int)x : -1;
    }
  };
  if constexpr (kList) {
    for (int i = threadIdx.x; i < (s1 - s0) * kGStep; i += kThreads)
      pos_all[i] = entry_pos(s0 * kGStep + i);
    __syncthreads();
  }

  // Q^T operand of this lane's row
  bf16x8 qb[C::KK];
  {
    const uint16_t* qp = (const uint16_t*)p.q + (((size_t)b * p.Tq + j) * p.Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++)
      qb[kk] = __builtin_bit_cast(bf16x8, row_ok ? *(const u32x4*)(qp + 32 * kk + 8 * jg)
                                                 : u32x4{0, 0, 0, 0});
  }

  // tile loads: thread chunk c = threadIdx.x + kThreads * i is row c / CPR, 16 bytes ch = c % CPR
  const int row_bytes = p.Hkv * D * 2;
  const size_t kv_row_stride = (size_t)p.Hkv * D;
  const uint16_t* kbase = (const uint16_t*)p.k + ((size_t)b * p.Tk * p.Hkv + u) * D;
  const uint16_t* vbase = (const uint16_t*)p.v + ((size_t)b * p.Tk * p.Hkv + u) * D;
  int voff[kPer];
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    const int c = threadIdx.x + kThreads * i;
    voff[i] = (c / C::CPR) * row_bytes + (c % C::CPR) * 16;
  }
  // list modes: one descriptor over this batch entry's rows of head u; a chunk's offset is its
  // entry's position, or past the end (reads zeros) for no position
  const int list_rec = (int)((long long)p.Tk * row_bytes - (long long)u * D * 2);
  auto list_off = [&](int s, int i) -> int {
    const int c = threadIdx.x + kThreads * i;
    const int e = (s - s0) * kGStep + c / C::CPR;
    const int pos = s < s1 ? pos_all[e] : -1;
    return pos >= 0 ? pos * row_bytes + (c % C::CPR) * 16 : 0x7FFFFFF0;
  };
  // range mode: descriptor of step s: its first row and the rows through t_row (past them:
  // zeros, masked); no rows at all for steps past this split (the prefetch runs two steps ahead)
  auto rsrc = [&](const uint16_t* base, int s) {
    const long long valid = s < s1 ? t_row + 1 - (long long)s * kGStep : 0;
    const int rows = valid < 0 ? 0 : (valid > kGStep ? kGStep : (int)valid);
    const int n_rec = __builtin_amdgcn_readfirstlane(rows * row_bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)s * kGStep * kv_row_stride), 0,
                                             n_rec, kBufferConfig);
  };
  // two register sets (the two steps after the one being computed are both in flight), or one
  // when a thread holds more than 8 chunks per step (2 waves, d 256: registers)
  constexpr int kSets = kPer <= 8 ? 2 : 1;
  u32x4 kreg[kSets][kPer], vreg[kSets][kPer];
  auto load = [&](int s, int set) {
    const auto rk = kList ? __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, list_rec, kBufferConfig)
                          : rsrc(kbase, s);
    const auto rv = kList ? __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, list_rec, kBufferConfig)
                          : rsrc(vbase, s);
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      if (kPer * kThreads == C::kChunks || threadIdx.x + kThreads * i < C::kChunks) {
        const int off = kList ? list_off(s, i) : voff[i];
        kreg[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
        vreg[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kNonTemporal));
      }
    }
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int c = threadIdx.x + kThreads * i;
      if (kPer * kThreads == C::kChunks || c < C::kChunks) {
        const int row = c / C::CPR, ch = c % C::CPR;
        *(u32x4*)&kt[buf][row * C::KStr + ch * 8] = kreg[set][i];
        *(u32x4*)&vt[buf][row * C::VStr + ch * 8] = vreg[set][i];
      }
    }
  };

  float m_run = -INFINITY;
  float l_s = 0.f, l_c = 0.f;
  f32x4 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  float* lrow = LOGITS ? p.logits + (((size_t)b * p.Tq + j) * p.Hq + h) * (size_t)p.Tk : nullptr;

  auto compute = [&](int s, int buf) {
    // S^T for this wave's 16-key blocks (keys kKeys * kh .. of the step)
    const int kw = kKeys * kh;
    f32x4 sacc[kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; kb++) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; kk++)
#pragma unroll
      for (int kb = 0; kb < kKB; kb++) {
        const bf16x8 ka = *(const bf16x8*)&kt[buf][(kw + 16 * kb + rn) * C::KStr + 32 * kk + 8 * jg];
        sacc[kb] = mfma_bf16(ka, qb[kk], sacc[kb]);
      }
    const int key0 = s * kGStep + kw;
    if (LOGITS && row_ok) {
#pragma unroll
      for (int kb = 0; kb < kKB; kb++) {
        const int e0 = key0 + 16 * kb + 4 * jg;
        if (p.logits_vec) {
          if (e0 < p.Tk) *(f32x4*)(lrow + e0) = sacc[kb];
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (e0 + e < p.Tk) lrow[e0 + e] = sacc[kb][e];
        }
      }
    }
    float sv[kKB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; kb++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int ke = kw + 16 * kb + 4 * jg + e;  // entry of the step
        const bool ok = kList ? pos_all[(s - s0) * kGStep + ke] >= 0
                              : (long long)s * kGStep + ke <= t_row;
        const float v = ok ? sacc[kb][e] * p.scale_log2 : -INFINITY;
        sv[kb][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = max4groups(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
    bf16x8 pb[kKB / 2];
#pragma unroll
    for (int half = 0; half < kKB / 2; half++) {
      float p8[8];
#pragma unroll
      for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float pe = fast_exp2(sv[2 * half + k2][e] - m_use);
          p8[4 * k2 + e] = pe;
          psum += pe;
        }
      pb[half] = pack_bf16x8(p8);
    }
    l_s *= alpha;
    l_c *= alpha;
    kahan_add(l_s, l_c, psum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::DB; db++) oacc[db] *= alpha;
    // O^T += V^T P^T, one MFMA per 32 keys (key blocks 2half, 2half + 1) and 16 columns
#pragma unroll
    for (int half = 0; half < kKB / 2; half++)
#pragma unroll
      for (int db = 0; db < C::DB; db++) {
        const uint16_t* a0 =
            &vt[buf][(kw + 32 * half + 4 * jg + (rn >> 2)) * C::VStr + 16 * db + 4 * (rn & 3)];
        const bf16x8 vop = join_tr(lds_read_tr16(a0), lds_read_tr16(a0 + 16 * C::VStr));
        oacc[db] = mfma_bf16(vop, pb[half], oacc[db]);
      }
  };

  // Step s is computed from LDS buffer (s - s0) & 1 while steps s + 1 and s + 2 are loading
  // into the register sets; two steps per loop trip keep the sets' roles fixed.  With one set,
  // only step s + 1 is loading.
  if (s0 < s1) {
    load(s0, 0);
    store(0, 0);
    lds_barrier();
    if constexpr (kSets == 2) {
      load(s0 + 1, 1);
      int s = s0;
      for (; s + 1 < s1; s += 2) {
        load(s + 2, 0);
        compute(s, 0);
        store(1, 1);  // step s + 1
        lds_barrier();
        load(s + 3, 1);
        compute(s + 1, 1);
        if (s + 2 < s1) store(0, 0);  // step s + 2
        lds_barrier();
      }
      if (s < s1) compute(s, 0);
    } else {
      for (int s = s0; s < s1; s++) {
        const int buf = (s - s0) & 1;
        load(s + 1, 0);
        compute(s, buf);
        if (s + 1 < s1) store(0, buf ^ 1);
        lds_barrier();
      }
    }
  }

  // row sum (the 4 lanes of the row summed)
  double ld = (double)l_s - (double)l_c;
  ld += __shfl_xor(ld, 16, 64);
  ld += __shfl_xor(ld, 32, 64);
  if constexpr (KH == 2) {
    // the second key half's maximum, row sum and O^T go through the (now free) V tiles, lane by
    // lane in the accumulator layout, to the first half's wave of the same head chunk
    static_assert(NW * (C::DB + 1) * 64 * 16 <= (int)sizeof(vt), "merge buffer");
    f32x4* xo = (f32x4*)&vt[0][0] + hc * (C::DB + 1) * 64;
    lds_barrier();  // every wave is done with the tiles
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < C::DB; db++) xo[db * 64 + lane] = oacc[db];
      const unsigned long long lb = (unsigned long long)__double_as_longlong(ld);
      xo[C::DB * 64 + lane] = f32x4{m_run, __uint_as_float((uint32_t)lb),
                                    __uint_as_float((uint32_t)(lb >> 32)), 0.f};
    }
    lds_barrier();
    if (kh == 1) return;
    // (elements converted by value: a bit cast applied to an element of a vector reads the
    // vector's first element here)
    const f32x4 x = xo[C::DB * 64 + lane];
    const float m1 = x[0];
    const double l1 = __longlong_as_double((long long)((unsigned long long)__float_as_uint(x[1]) |
                                                       ((unsigned long long)__float_as_uint(x[2]) << 32)));
    const float M = fmaxf(m_run, m1);
    const float f0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
    const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
    ld = (m_run == -INFINITY ? 0.0 : exp2((double)m_run - (double)M) * ld) +
         (m1 == -INFINITY ? 0.0 : exp2((double)m1 - (double)M) * l1);
#pragma unroll
    for (int db = 0; db < C::DB; db++) oacc[db] = oacc[db] * f0 + xo[db * 64 + lane] * f1;
    m_run = M;
  }
  if (p.final_direct) {  // one split: normalize here (sink, output gate) and write O and LSE
    if (!row_ok) return;
    const size_t orow = ((size_t)b * p.Tq + j) * p.Hq + h;
    const bool ch = p.gate_ch && p.out_gate;  // per-channel output gate
    const RowNorm n = row_norm(m_run, ld, p.sink, h, ch ? 1.0 : out_gate_of(p.out_gate, orow));
#pragma unroll
    for (int db = 0; db < C::DB; db++) {
      const int c0 = 16 * db + 4 * jg;  // this lane's 4 columns of row rn
      float o4[4];
#pragma unroll
      for (int e = 0; e < 4; e++)
        o4[e] = oacc[db][e] * n.factor * (ch ? sigmoid_f(p.out_gate[orow * D + c0 + e]) : 1.f);
      if (p.out_f32) {
        *(f32x4*)((float*)p.o + orow * D + c0) = f32x4{o4[0], o4[1], o4[2], o4[3]};
      } else {
        uint16_t* op = (uint16_t*)p.o + orow * D + c0;
        const uint32_t lo = (uint32_t)f2bf(o4[0]) | ((uint32_t)f2bf(o4[1]) << 16);
        const uint32_t hi = (uint32_t)f2bf(o4[2]) | ((uint32_t)f2bf(o4[3]) << 16);
        *(uint2*)op = make_uint2(lo, hi);
      }
    }
    if (p.lse && jg == 0) p.lse[((size_t)b * p.Hq + h) * p.Tq + j] = n.lse;
    return;
  }
  // partials of this split: row maximum, row sum, O^T
  const size_t n_sets = (size_t)p.B * p.Hkv * p.sets_per_bu * p.cpq;
  const int set = ((b * p.Hkv + u) * p.sets_per_bu + j) * p.cpq + hc;
  const size_t prow = ((size_t)split * n_sets + set) * 16 + rn;
  if (jg == 0) {
    p.part_m[prow] = m_run;
    p.part_l[prow] = ld;
  }
#pragma unroll
  for (int db = 0; db < C::DB; db++) *(f32x4*)(p.part_o + prow * D + 16 * db + 4 * jg) = oacc[db];
}

template <int D, int NW>
hipError_t launch_nw(const RowAttnParams& p, KeySrc src, hipStream_t stream) {
  const dim3 grid(p.n_split * p.B * p.Hkv * p.Tq);
  constexpr int kListThreads = 64 * NW * key_halves<D, NW, SRC_TOKEN>();
  constexpr int kRangeThreads = 64 * NW * key_halves<D, NW, SRC_RANGE>();
  if (src == SRC_TOKEN)
    group_attn_kernel<D, NW, SRC_TOKEN, false><<<grid, kListThreads, 0, stream>>>(p);
  else if (src == SRC_BLOCK)
    group_attn_kernel<D, NW, SRC_BLOCK, false><<<grid, kListThreads, 0, stream>>>(p);
  else if (p.logits)
    group_attn_kernel<D, NW, SRC_RANGE, true><<<grid, kRangeThreads, 0, stream>>>(p);
  else
    group_attn_kernel<D, NW, SRC_RANGE, false><<<grid, kRangeThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const RowAttnParams& p, KeySrc src, hipStream_t stream) {
  switch (p.cpq) {
    case 2: return launch_nw<D, 2>(p, src, stream);
    case 3: return launch_nw<D, 3>(p, src, stream);
    case 4: return launch_nw<D, 4>(p, src, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_group_attn(const RowAttnParams& p, int head_dim, KeySrc src, hipStream_t stream) {
  if (p.hpc != 16 || p.q_per_set != 1 || p.sets_per_bu != p.Tq || p.n_split < 1 || p.pages)
    return hipErrorInvalidValue;
  if (src == SRC_WINDOW || (src != SRC_RANGE && p.logits)) return hipErrorInvalidValue;
  if (src != SRC_RANGE && p.steps_per_split * kGStep > kMaxSplitEntries) return hipErrorInvalidValue;
  if (head_dim == 256) return launch_d<256>(p, src, stream);
  if (head_dim == 128) return launch_d<128>(p, src, stream);
  return hipErrorInvalidValue;
}

}  // namespace hs
