// abi.cpp -- the C ABI (include/hysparse.h): host-side validation, workspace layout and the
// choice of launch geometry.  No kernel is enqueued before every argument has been checked.
#include "hysparse.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "hs_kernels.h"

namespace {

// Finite float test on the bit pattern: this file is built with -fno-honor-nans (for the
// kernels' max operations), under which comparisons may assume that no operand is NaN.
bool finite_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return (u & 0x7F800000u) != 0x7F800000u;
}

thread_local char g_err[512] = "";

hs_status fail(hs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

hs_status ok() {
  g_err[0] = 0;
  return HS_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Resolved shape of a call.
struct Shape {
  int B, Tq, Tk, Hq, Hkv, D, g;
  long long q_off;
  bool in_f32, out_f32;
  float scale_log2;  // logit scale times log2(e): the kernels work in base 2
};

hs_status check_desc(const hs_attn_desc* d, Shape* s) {
  if (!d) return fail(HS_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1 || d->q_len < 1 || d->kv_len < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(HS_ERR_INVALID_ARG, "batch, q_len, kv_len and head counts must be >= 1");
  if (d->n_q_heads % d->n_kv_heads)
    return fail(HS_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                d->n_q_heads, d->n_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(HS_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128 or 256)", d->head_dim);
  if ((d->in_dtype != HS_BF16 && d->in_dtype != HS_F32) ||
      (d->out_dtype != HS_BF16 && d->out_dtype != HS_F32))
    return fail(HS_ERR_INVALID_ARG, "unknown dtype");
  long long q_off = d->q_offset == -1 ? (long long)d->kv_len - d->q_len : d->q_offset;
  if (q_off < 0 || q_off + d->q_len > d->kv_len)
    return fail(HS_ERR_INVALID_ARG, "q_offset %lld with q_len %d does not fit kv_len %d", q_off,
                d->q_len, d->kv_len);
  if (!finite_bits(d->scale) || d->scale < 0.f)
    return fail(HS_ERR_INVALID_ARG, "scale %g: must be finite and >= 0 (0: 1/sqrt(head_dim))",
                (double)d->scale);
  const int g = d->n_q_heads / d->n_kv_heads;
  if (g > 64)
    return fail(HS_ERR_UNSUPPORTED, "GQA group of %d query heads per KV head (at most 64)", g);
  // 32-bit position arithmetic inside the kernels
  if ((long long)d->kv_len > (1LL << 30))
    return fail(HS_ERR_UNSUPPORTED, "kv_len %d too large", d->kv_len);
  s->B = d->batch;
  s->Tq = d->q_len;
  s->Tk = d->kv_len;
  s->Hq = d->n_q_heads;
  s->Hkv = d->n_kv_heads;
  s->D = d->head_dim;
  s->g = g;
  s->q_off = q_off;
  s->in_f32 = d->in_dtype == HS_F32;
  s->out_f32 = d->out_dtype == HS_F32;
  const double tau = d->scale > 0.f ? (double)d->scale : 1.0 / std::sqrt((double)d->head_dim);
  s->scale_log2 = (float)(1.4426950408889634 * tau);
  return HS_OK;
}

// ---- row-attention geometry ----------------------------------------------------------------
constexpr int kStepKeys = 32;
constexpr int kTargetWorkgroups = 2048;

struct RaGeom {
  int q_per_set, sets_per_bu, n_sets, n_split, steps_per_split;
};

// Splits of each row-set's key list: enough workgroups to fill the GPU (`target`), no split
// shorter than `min_steps` 32-key steps, none longer than `max_steps`.
// Heads per row-set and head chunks per query: groups of more than 16 heads run as chunks of 16.
int heads_per_set(const Shape& s) { return s.g < 16 ? s.g : 16; }
int chunks_per_query(const Shape& s) { return (s.g + heads_per_set(s) - 1) / heads_per_set(s); }

RaGeom ra_geom(const Shape& s, bool per_query, long long max_keys, int min_steps_per_split,
               long long target = kTargetWorkgroups, long long max_steps = 1LL << 40) {
  RaGeom g;
  g.q_per_set = per_query ? 1 : 16 / heads_per_set(s);
  g.sets_per_bu = (s.Tq + g.q_per_set - 1) / g.q_per_set;
  g.n_sets = s.B * s.Hkv * g.sets_per_bu * chunks_per_query(s);
  const long long steps = (max_keys + kStepKeys - 1) / kStepKeys;
  long long want = (target + g.n_sets - 1) / g.n_sets;
  long long most = (steps + min_steps_per_split - 1) / min_steps_per_split;
  if (want > most) want = most;
  const long long least = (steps + max_steps - 1) / max_steps;
  if (want < least) want = least;
  if (want < 1) want = 1;
  g.steps_per_split = (int)((steps + want - 1) / want);
  if (g.steps_per_split < 1) g.steps_per_split = 1;
  g.n_split = (int)((steps + g.steps_per_split - 1) / g.steps_per_split);
  if (g.n_split < 1) g.n_split = 1;
  return g;
}

size_t partial_bytes(const RaGeom& g, int D) {
  const size_t rows = (size_t)g.n_split * g.n_sets * 16;
  return align_up(rows * 4, 256) + align_up(rows * 8, 256) + align_up(rows * 4 * D, 256);
}

void carve_partials(void* base, const RaGeom& g, int D, float** m, double** l, float** o) {
  const size_t rows = (size_t)g.n_split * g.n_sets * 16;
  char* p = (char*)base;
  *m = (float*)p;
  p += align_up(rows * 4, 256);
  *l = (double*)p;
  p += align_up(rows * 8, 256);
  *o = (float*)p;
}

hs::RowAttnParams ra_params(const Shape& s, const RaGeom& g) {
  hs::RowAttnParams p;
  memset(&p, 0, sizeof(p));
  p.B = s.B;
  p.Tq = s.Tq;
  p.Tk = s.Tk;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = s.g;
  p.hpc = heads_per_set(s);
  p.cpq = chunks_per_query(s);
  p.q_off = s.q_off;
  p.q_per_set = g.q_per_set;
  p.sets_per_bu = g.sets_per_bu;
  p.n_split = g.n_split;
  p.steps_per_split = g.steps_per_split;
  p.scale_log2 = s.scale_log2;
  p.out_f32 = s.out_f32;
  return p;
}

hs::CombineParams combine_params(const Shape& s, const RaGeom& g, void* o, float* lse) {
  hs::CombineParams c;
  memset(&c, 0, sizeof(c));
  c.B = s.B;
  c.Tq = s.Tq;
  c.Hq = s.Hq;
  c.Hkv = s.Hkv;
  c.g = s.g;
  c.hpc = heads_per_set(s);
  c.cpq = chunks_per_query(s);
  c.q_per_set = g.q_per_set;
  c.sets_per_bu = g.sets_per_bu;
  c.o = o;
  c.lse = lse;
  c.out_f32 = s.out_f32;
  return c;
}

hs_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- full attention ------------------------------------------------------------------------
constexpr long long kResidentWorkgroups = 512;  // 256 CUs x 2 workgroups of this kernel

// Many queries per KV head (bf16): the LDS-tiled prefill kernel; otherwise the row kernel.
// (A group of more than 16 heads needs at least 128 rows per KV head to fill half a workgroup;
// with fewer, the row kernel's key splits do better.)
// (Head size 256 runs 128 rows per workgroup, smaller heads 256: the group must divide them.)
bool use_prefill_kernel(const Shape& s) {
  const long long rows = (long long)s.Tq * s.g;
  const int rows_wg = s.D > 128 ? 128 : 256;
  return !s.in_f32 && rows > 16 && (s.g <= 16 || rows >= 128) && rows_wg % s.g == 0;
}

// Kernels that read Q, K, V take head_dim 256 with bf16 inputs only.
hs_status check_qkv_dtype(const Shape& s) {
  if (s.D == 256 && s.in_f32) return fail(HS_ERR_UNSUPPORTED, "head_dim 256 needs bf16 inputs");
  return HS_OK;
}

size_t row_fa_ws(const Shape& s, int page_size);
size_t full_attn_ws(const Shape& s) {
  if (use_prefill_kernel(s)) return 0;
  return row_fa_ws(s, 0);
}

// ---- token top-k ---------------------------------------------------------------------------
struct TkGeom {
  int q_per_set, sets_per_bu, n_split, keys_per_split, sel_split, keys_per_sel;
  size_t rows;
};

TkGeom tk_geom(const Shape& s) {
  TkGeom t;
  t.q_per_set = s.g <= 16 ? 16 / s.g : 1;  // query rows packed per 16-row score set
  t.sets_per_bu = (s.Tq + t.q_per_set - 1) / t.q_per_set;
  const long long n_sets = (long long)s.B * s.Hkv * t.sets_per_bu;
  // four workgroups per resident slot: measured 5 us faster than one round on the 7B decode step
  long long want = (4 * kResidentWorkgroups + n_sets - 1) / n_sets;
  const long long most = (s.Tk + 255) / 256;
  if (want > most) want = most;
  if (want < 1) want = 1;
  long long kps = (s.Tk + want - 1) / want;
  kps = (kps + 63) / 64 * 64;
  t.keys_per_split = (int)kps;
  t.n_split = (int)((s.Tk + kps - 1) / kps);
  t.rows = (size_t)s.B * s.Tq * s.Hkv;
  // selection passes: chunks of at least 8192 keys, enough chunks to fill the GPU
  long long ks = 8192;
  while (ks > 1024 && (long long)t.rows * ((s.Tk + ks - 1) / ks) < 512) ks /= 2;
  while ((s.Tk + ks - 1) / ks > 4096) ks *= 2;
  t.keys_per_sel = (int)ks;
  t.sel_split = (int)((s.Tk + ks - 1) / ks);
  return t;
}

struct TkLayout {
  size_t keys, hist, blist, above, counts, state, total;
};

TkLayout tk_layout(const Shape& s, const TkGeom& t) {
  TkLayout L;
  size_t o = 0;
  L.keys = o;
  o += align_up(t.rows * (size_t)s.Tk * 4, 256);
  L.hist = o;  // histograms, then the boundary counters (zeroed together)
  o += align_up((t.rows * 2048 + t.rows) * 4, 256);
  // the rest only for rows long enough to take the multi-kernel chain
  const bool chain = hs::topk_decode_uses_chain(s.Tk);
  L.blist = o;
  o += chain ? align_up(t.rows * (size_t)s.Tk * 8, 256) : 0;
  L.above = o;
  o += chain ? align_up(t.rows * (size_t)t.sel_split * 4, 256) : 0;
  L.counts = o;
  o += chain ? align_up(t.rows * (size_t)t.sel_split * 4, 256) : 0;
  L.state = o;
  o += chain ? align_up(t.rows * 2 * 4, 256) : 0;
  L.total = o;
  return L;
}

size_t tk_ws(const Shape& s, const TkGeom& t) { return tk_layout(s, t).total; }

// Token selection from stored logits: one (b, t, u) row per workgroup and key chunk (chunks of
// whole 1024-key passes: a thread reads 4 consecutive keys of every head per pass); the
// selection passes are those of tk_geom.
TkGeom tl_geom(const Shape& s) {
  TkGeom t = tk_geom(s);
  t.q_per_set = 1;
  t.sets_per_bu = s.Tq;
  long long want = (1024 + (long long)t.rows - 1) / (long long)t.rows;
  const long long most = (s.Tk + 1023) / 1024;
  if (want > most) want = most;
  if (want < 1) want = 1;
  long long kps = (s.Tk + want - 1) / want;
  kps = (kps + 1023) / 1024 * 1024;
  t.keys_per_split = (int)kps;
  t.n_split = (int)((s.Tk + kps - 1) / kps);
  return t;
}

// Decode-path parameters of the token selection (score pass from Q, K or from stored logits).
hs::TopkDecodeParams tk_params(const Shape& s, const TkGeom& t, const float* lse, int k_global,
                               int window, int32_t* idx, int32_t* count, void* ws) {
  hs::TopkDecodeParams p;
  memset(&p, 0, sizeof(p));
  p.lse = lse;
  p.B = s.B;
  p.Tq = s.Tq;
  p.Tk = s.Tk;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = s.g;
  p.q_off = s.q_off;
  p.k_global = k_global;
  p.window = window;
  p.q_per_set = t.q_per_set;
  p.sets_per_bu = t.sets_per_bu;
  p.n_split = t.n_split;
  p.keys_per_split = t.keys_per_split;
  p.sel_split = t.sel_split;
  p.keys_per_sel = t.keys_per_sel;
  p.scale_log2 = s.scale_log2;
  const TkLayout lay = tk_layout(s, t);
  char* w = (char*)ws;
  p.keys = (uint32_t*)(w + lay.keys);
  p.hist = (uint32_t*)(w + lay.hist);
  p.bcount = p.hist + t.rows * 2048;
  p.blist = (unsigned long long*)(w + lay.blist);
  p.above = (uint32_t*)(w + lay.above);
  p.counts = (uint32_t*)(w + lay.counts);
  p.state = (uint32_t*)(w + lay.state);
  p.idx = idx;
  p.cnt = count;
  p.cap = k_global + window;
  return p;
}

// Group sizes and head sizes the streamed prefill selection takes: groups of up to 16 heads sit
// in the rows of one 256-row tile (padded to 4, 8 or 16 heads); larger groups select per chunk
// of 16 heads and merge the chunks' candidates.
bool prefill_select_shape(const Shape& s) { return s.g <= 64 && (s.D <= 128 || !s.in_f32); }
int select_chunks(const Shape& s) { return s.g <= 16 ? 1 : (s.g + 15) / 16; }
size_t select_chunk_rows(const Shape& s) {
  return (size_t)s.B * s.Tq * s.Hkv * select_chunks(s);
}

bool logits_fit(const Shape& s);

// Many query rows per KV head: selection streams over K tiles and stores no per-key score.
// Chunked groups (above 16 heads) need 16 queries to fill a tile's rows; with fewer, computed
// logits serve them unless those would be too large.
bool use_prefill_select(const Shape& s, int k_global) {
  if (!prefill_select_shape(s) || k_global > hs::prefill_select_max_k()) return false;
  if (s.g <= 16) return (long long)s.Tq * s.g > 16;
  return s.Tq >= 16 || !logits_fit(s);
}

// The fused decode score passes (score, key and histogram in one kernel over K tiles).
bool fused_decode_score(const Shape& s) {
  return (s.g == 4 || s.g == 8 || s.g == 16) && s.D <= 128;
}

// Selection for every other shape with few query rows: the raw logits of the rows are computed
// into the workspace first, then selected like stored logits.  Bounded by their size.
constexpr size_t kMaxLogitBytes = (size_t)8 << 30;
size_t logit_bytes(const Shape& s) {
  return align_up((size_t)s.B * s.Tq * s.Hq * (size_t)s.Tk * 4, 256);
}
bool logits_fit(const Shape& s) { return logit_bytes(s) <= kMaxLogitBytes; }

hs::LogitsParams logits_params(const Shape& s, const void* q, const void* k, float* logits) {
  hs::LogitsParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.B = s.B;
  p.Tq = s.Tq;
  p.Tk = s.Tk;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = s.g;
  p.q_off = s.q_off;
  p.logits = logits;
  // key chunks of multiples of 256 keys, enough workgroups to fill the GPU
  const long long wgs = (long long)s.B * s.Tq * s.Hkv * ((s.g + 15) / 16);
  const long long keys = s.q_off + s.Tq;  // the longest row
  long long want = (2048 + wgs - 1) / wgs;
  const long long most = (keys + 255) / 256;
  if (want > most) want = most;
  if (want < 1) want = 1;
  long long kps = (keys + want - 1) / want;
  kps = (kps + 255) / 256 * 256;
  p.keys_per_split = (int)kps;
  p.n_split = (int)((keys + kps - 1) / kps);
  return p;
}

enum SelRoute { SEL_NONE, SEL_PREFILL, SEL_DECODE, SEL_LOGITS };

// candidate buffers of the (chunk) rows, then, with chunks, their kept counts
size_t tk_prefill_ws(const Shape& s) {
  const size_t rows = select_chunk_rows(s);
  const size_t buf = align_up(rows * hs::prefill_select_buffer_cap() * 8, 256);
  return buf + (select_chunks(s) > 1 ? align_up(rows * 4, 256) : 0);
}

// block mode: nothing for a whole group; with chunks, their kept values and counts
size_t bk_prefill_ws(const Shape& s, int n_blocks) {
  if (select_chunks(s) == 1) return 0;
  const size_t rows = select_chunk_rows(s);
  return align_up(rows * (size_t)n_blocks * 8, 256) + align_up(rows * 4, 256);
}

hs::PrefillSelectParams select_params(const Shape& s, const void* q, const void* k,
                                      const float* lse) {
  hs::PrefillSelectParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.lse = lse;
  p.B = s.B;
  p.Tq = s.Tq;
  p.Tk = s.Tk;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = s.g;
  p.q_off = s.q_off;
  p.scale_log2 = s.scale_log2;
  p.chunks = select_chunks(s);
  return p;
}

// ---- block top-k ---------------------------------------------------------------------------
struct BkGeom {
  int q_per_set, sets_per_bu, n_split, blocks_per_split;
  size_t rows;
};

BkGeom bk_geom(const Shape& s, int block, int n_blocks, bool per_row = false) {
  BkGeom t;
  t.q_per_set = (per_row || s.g > 16) ? 1 : 16 / s.g;  // query rows per 16-row score set
  t.sets_per_bu = (s.Tq + t.q_per_set - 1) / t.q_per_set;
  const long long n_sets = (long long)s.B * s.Hkv * t.sets_per_bu;
  const long long nblk = (s.Tk + block - 1) / block;
  // fewer, longer splits than the token path: the merge cost grows with splits * n_blocks
  long long want = (kResidentWorkgroups + n_sets - 1) / n_sets;
  const long long most = (nblk + 3) / 4;
  if (want > most) want = most;
  const long long least = (nblk + 255) / 256;  // at most 256 blocks per workgroup
  if (want < least) want = least;
  if (want < 1) want = 1;
  long long bps = (nblk + want - 1) / want;
  t.blocks_per_split = (int)bps;
  t.n_split = (int)((nblk + bps - 1) / bps);
  t.rows = (size_t)s.B * s.Tq * s.Hkv;
  return t;
}

// per_row: selection from logits (stored or computed; one (b, t, u) row per workgroup and
// split, any group size)
hs_status bk_check(const Shape& s, int block, int n_blocks, BkGeom* g, bool per_row = false) {
  if (block < 16 || block % 16) return fail(HS_ERR_UNSUPPORTED, "block %d: must be a multiple of 16", block);
  if (n_blocks < 1 || n_blocks > 64) return fail(HS_ERR_UNSUPPORTED, "n_blocks %d: must be 1..64", n_blocks);
  *g = bk_geom(s, block, n_blocks, per_row);
  if ((long long)g->n_split * n_blocks > 4096)
    return fail(HS_ERR_UNSUPPORTED, "context too long for the block merge (%d splits)", g->n_split);
  return HS_OK;
}

// Many query rows per KV head and blocks that tile 64 keys: streamed running top-n.
bool use_prefill_blocks(const Shape& s, int block) {
  if (64 % block || !prefill_select_shape(s)) return false;
  if (s.g <= 16) return (long long)s.Tq * s.g > 16;
  return s.Tq >= 16 || !logits_fit(s);
}

size_t bk_ws(const BkGeom& g, int n_blocks) {
  return align_up(g.rows * (size_t)g.n_split * n_blocks * 8, 256);
}

// Route of a token selection from Q and K.
SelRoute token_route(const Shape& s, int k_global) {
  if (use_prefill_select(s, k_global)) return SEL_PREFILL;
  if (fused_decode_score(s)) return SEL_DECODE;
  if (logits_fit(s)) return SEL_LOGITS;
  return SEL_NONE;
}

// Route of a block selection from Q and K, with its merge geometry.
hs_status block_route(const Shape& s, int block, int n_blocks, SelRoute* r, BkGeom* g) {
  hs_status st = bk_check(s, block, n_blocks, g);
  if (st != HS_OK) return st;
  if (use_prefill_blocks(s, block)) {
    *r = SEL_PREFILL;
  } else if (fused_decode_score(s)) {
    *r = SEL_DECODE;
  } else if (logits_fit(s)) {
    *r = SEL_LOGITS;
    return bk_check(s, block, n_blocks, g, true);
  } else {
    *r = SEL_NONE;
    return fail(HS_ERR_UNSUPPORTED, "block selection: %zu bytes of logits for this shape exceed "
                "the %zu-byte bound of the route for this group and head size", logit_bytes(s),
                kMaxLogitBytes);
  }
  return HS_OK;
}

size_t block_select_ws(SelRoute r, const Shape& s, const BkGeom& g, int n_blocks) {
  if (r == SEL_PREFILL) return bk_prefill_ws(s, n_blocks);
  if (r == SEL_LOGITS) return logit_bytes(s) + bk_ws(g, n_blocks);
  return bk_ws(g, n_blocks);
}

// ---- sparse attention ----------------------------------------------------------------------
struct SparseGeom {
  RaGeom glob, loc;
  bool wide;     // few row-sets: one 8-wave workgroup per set instead of split key lists
  bool combine;  // split partials merged by the combine kernel
  bool fused;    // gated layer with unsplit branches: both in one workgroup, no partials
  bool group;    // the global branch on the group kernel (groups of more than 16 heads)
};

bool use_group_kernel(const Shape& s, bool paged);
RaGeom group_list_geom(const Shape& s, long long keys_per_set);

// The group kernel addresses a batch entry's K / V rows with 32-bit byte offsets.
bool group_list_fits(const Shape& s) {
  return (long long)s.Tk * s.Hkv * s.D * 2 < (1LL << 31);
}

SparseGeom sparse_geom(const Shape& s, long long keys_per_set, int window, bool paged = false) {
  SparseGeom g;
  g.group = use_group_kernel(s, paged) && group_list_fits(s);
  if (g.group) {
    g.glob = group_list_geom(s, keys_per_set);
    g.wide = false;
    g.fused = false;
    g.loc = ra_geom(s, true, window > 0 ? window : 1, 4);
    // unsplit lists without a window branch: the group kernel writes the output itself
    g.combine = window > 0 || g.glob.n_split > 1;
    return g;
  }
  g.glob = ra_geom(s, true, keys_per_set, 4, kTargetWorkgroups, 64);
  // Decode-sized index sets (at most 64 steps of 32 keys): rather than splitting each list over
  // several workgroups and merging partials in a second kernel, one workgroup of 8 waves takes
  // the whole list of its set and writes the final output.  Measured on the 7B decode shape
  // (1152 keys per set): 5.3 TB/s at 1024 sets against 3.9 TB/s split; below about 96 sets the
  // work is latency-bound and the split version is slightly faster.
  const long long n_sets = (long long)g.glob.n_sets;
  g.wide = !s.in_f32 && s.D <= 128 && g.glob.n_split > 1 && keys_per_set <= 64LL * kStepKeys &&
           n_sets >= 96;
  if (g.wide) {
    g.glob.steps_per_split = (int)((keys_per_set + kStepKeys - 1) / kStepKeys);
    g.glob.n_split = 1;
  }
  g.loc = ra_geom(s, true, window > 0 ? window : 1, 4);
  g.fused = window > 0 && s.D <= 128 && g.glob.n_split == 1 && g.loc.n_split == 1;
  g.combine = !g.fused && (window > 0 || g.glob.n_split > 1);
  return g;
}

size_t sparse_ws(const Shape& s, const SparseGeom& g, int window) {
  if (!g.combine) return 0;
  size_t b = partial_bytes(g.glob, s.D);
  if (window > 0) b += partial_bytes(g.loc, s.D);
  return b;
}

// Geometry of full attention on the row kernel.  Paged K / V: a split's pages are staged in LDS,
// so no split may span more than kMaxStagedPages of them.
constexpr long long kMaxStagedPages = 2048;
RaGeom fa_row_geom(const Shape& s, int page_size) {
  long long max_steps = 1LL << 40;
  if (page_size > 0) max_steps = ((kMaxStagedPages - 1) * page_size) / kStepKeys;
  if (max_steps < 1) max_steps = 1;
  return ra_geom(s, false, s.q_off + s.Tq, 8, kResidentWorkgroups, max_steps);
}

// Groups of more than 16 heads per KV head (bf16, contiguous K / V): the group kernel, one
// workgroup per (batch entry, KV head, query, key split) whose waves are the 16-head chunks and
// share every 64-key step of K / V through LDS.  It always writes split partials.
constexpr int kGroupStepKeys = 64;
bool use_group_kernel(const Shape& s, bool paged) {
  return s.g > 16 && !s.in_f32 && (s.D == 128 || s.D == 256) && !paged;
}

RaGeom group_geom(const Shape& s) {
  RaGeom g;
  g.q_per_set = 1;
  g.sets_per_bu = s.Tq;
  g.n_sets = s.B * s.Hkv * s.Tq * chunks_per_query(s);
  const long long steps = (s.q_off + s.Tq + kGroupStepKeys - 1) / kGroupStepKeys;
  const long long wgs = (long long)s.B * s.Hkv * s.Tq;
  const long long target = s.D == 256 ? 256 : 512;  // LDS: one (d 256) or two workgroups per CU
  long long want = (target + wgs - 1) / wgs;
  const long long most = (steps + 7) / 8;  // no split shorter than 8 steps
  if (want > most) want = most;
  if (want < 1) want = 1;
  g.steps_per_split = (int)((steps + want - 1) / want);
  g.n_split = (int)((steps + g.steps_per_split - 1) / g.steps_per_split);
  return g;
}

// Index lists on the group kernel: 64-entry steps, at most 32 per split (staged in LDS), enough
// workgroups to fill the GPU.
RaGeom group_list_geom(const Shape& s, long long keys_per_set) {
  RaGeom g;
  g.q_per_set = 1;
  g.sets_per_bu = s.Tq;
  g.n_sets = s.B * s.Hkv * s.Tq * chunks_per_query(s);
  const long long steps = (keys_per_set + kGroupStepKeys - 1) / kGroupStepKeys;
  const long long wgs = (long long)s.B * s.Hkv * s.Tq;
  const long long target = s.D == 256 ? 256 : 512;
  long long want = (target + wgs - 1) / wgs;
  if (want > steps) want = steps;
  const long long least = (steps + 31) / 32;
  if (want < least) want = least;
  if (want < 1) want = 1;
  g.steps_per_split = (int)((steps + want - 1) / want);
  if (g.steps_per_split < 1) g.steps_per_split = 1;
  g.n_split = (int)((steps + g.steps_per_split - 1) / g.steps_per_split);
  if (g.n_split < 1) g.n_split = 1;
  return g;
}

// Workspace of full attention on the row path (decode, short query blocks, stored logits,
// paged caches).
size_t row_fa_ws(const Shape& s, int page_size) {
  if (use_group_kernel(s, page_size > 0)) {
    const RaGeom g = group_geom(s);
    return g.n_split > 1 ? partial_bytes(g, s.D) : 0;
  }
  const RaGeom g = fa_row_geom(s, page_size);
  return g.n_split > 1 ? partial_bytes(g, s.D) : 0;
}

// Pages of the paged selection calls hold whole 64-key tiles of the streamed selection.
constexpr int kPagedSelectMinPage = 64;

// Paged full attention of a prefill shape without stored logits runs on the tiled prefill
// kernel when a page holds whole key tiles; everything else on the row kernel.
bool paged_prefill_attn(const Shape& s, bool with_logits, int page_size) {
  return !with_logits && use_prefill_kernel(s) && page_size >= hs::prefill_tile_keys(s.D);
}

hs_status check_pages(const Shape& s, const hs_kv_pages* pg) {
  if (!pg || !pg->block_table) return fail(HS_ERR_INVALID_ARG, "NULL page table");
  const int P = pg->page_size;
  if (P < 1 || (P & (P - 1)) || P > (1 << 20))
    return fail(HS_ERR_INVALID_ARG, "page_size %d: must be a power of two (1 .. 2^20)", P);
  if (pg->n_pages < 1) return fail(HS_ERR_INVALID_ARG, "n_pages must be >= 1");
  if ((long long)pg->max_pages * P < s.Tk)
    return fail(HS_ERR_INVALID_ARG, "max_pages %d x page_size %d < kv_len %d", pg->max_pages, P,
                s.Tk);
  if ((long long)pg->n_pages * P * s.Hkv * s.D > (1LL << 40))
    return fail(HS_ERR_UNSUPPORTED, "page pool too large");
  return HS_OK;
}

void set_pages(hs::RowAttnParams& p, const hs_kv_pages* pg) {
  p.pages = pg->block_table;
  p.page_size = pg->page_size;
  p.max_pages = pg->max_pages;
  p.n_pages = pg->n_pages;
}

// Full attention on the row kernel (decode and short query blocks); logits != nullptr also
// stores every computed dot product q.k to logits [B, Tq, Hq, Tk].
hs_status row_full_attn(const Shape& s, const void* q, const void* k, const void* v, void* o,
                        float* lse, float* logits, void* ws, size_t ws_bytes, void* stream,
                        const hs_kv_pages* pages = nullptr) {
  const bool group = use_group_kernel(s, pages != nullptr);
  const RaGeom g = group ? group_geom(s) : fa_row_geom(s, pages ? pages->page_size : 0);
  const size_t need = row_fa_ws(s, pages ? pages->page_size : 0);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hs::RowAttnParams p = ra_params(s, g);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.logits = logits;
  p.logits_vec = logits && s.Tk % 4 == 0 && (uintptr_t)logits % 16 == 0;
  if (pages) set_pages(p, pages);
  p.final_direct = g.n_split == 1;
  if (!p.final_direct) carve_partials(ws, g, s.D, &p.part_m, &p.part_l, &p.part_o);
  hipStream_t hst = (hipStream_t)stream;
  hipError_t e = group ? hs::launch_group_attn(p, s.D, hs::SRC_RANGE, hst)
                       : hs::launch_row_attn(p, s.D, s.in_f32, hs::SRC_RANGE, hst);
  if (e != hipSuccess) return hip_status(e, "full attention kernel");
  if (!p.final_direct) {
    hs::CombineParams c = combine_params(s, g, o, lse);
    c.n_branch = 1;
    c.m[0] = p.part_m;
    c.l[0] = p.part_l;
    c.po[0] = p.part_o;
    c.n_split[0] = g.n_split;
    e = hs::launch_combine(c, s.D, hst);
    if (e != hipSuccess) return hip_status(e, "combine kernel");
  }
  return ok();
}

hs::PrefillParams prefill_params(const Shape& s, const void* q, const void* k, const void* v,
                                 void* o, float* lse) {
  hs::PrefillParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q = q;
  pp.k = k;
  pp.v = v;
  pp.B = s.B;
  pp.Tq = s.Tq;
  pp.Tk = s.Tk;
  pp.Hq = s.Hq;
  pp.Hkv = s.Hkv;
  pp.g = s.g;
  pp.q_off = s.q_off;
  pp.scale_log2 = s.scale_log2;
  pp.o = o;
  pp.lse = lse;
  pp.out_f32 = s.out_f32;
  return pp;
}

// Block selection inside the prefill attention pass: blocks of one 64-key tile, at most 16
// blocks per list.
bool fused_blocks(const Shape& s, int block, int n_blocks) {
  return use_prefill_kernel(s) && s.D <= 128 && 32 % s.g == 0 && block == 64 && n_blocks >= 1 &&
         n_blocks <= 16;
}

// Workspace of hs_full_attn_block_topk: none when fused, else what the larger of its two
// passes needs (they run one after the other and share it).
size_t fused_blocks_ws(const Shape& s, int block, int n_blocks) {
  if (fused_blocks(s, block, n_blocks)) return 0;
  BkGeom g;
  SelRoute r;
  if (block_route(s, block, n_blocks, &r, &g) != HS_OK) return 0;
  const size_t a = full_attn_ws(s);
  const size_t b = block_select_ws(r, s, g, n_blocks);
  return a > b ? a : b;
}

// Workspace of a token selection from Q and K on its route (0 and an error: no route).
size_t token_select_ws(const Shape& s, int k_global) {
  switch (token_route(s, k_global)) {
    case SEL_PREFILL: return tk_prefill_ws(s);
    case SEL_DECODE: return tk_ws(s, tk_geom(s));
    case SEL_LOGITS: return logit_bytes(s) + tk_ws(s, tl_geom(s));
    case SEL_NONE: break;
  }
  fail(HS_ERR_UNSUPPORTED, "token selection: no route for this shape");
  return 0;
}

// Token selection started at the tile-maximum bound: the tiled prefill attention kernel (head
// sizes up to 128) and the streamed prefill selection (whole groups, or chunks of 16 heads).
bool fused_tokens(const Shape& s, int k_global) {
  return use_prefill_kernel(s) && s.D <= 128 && k_global >= 1 &&
         token_route(s, k_global) == SEL_PREFILL;
}
int tmax_stride(const Shape& s) {
  const long long bn = hs::prefill_tile_keys(s.D);
  const long long tiles = (s.Tk + bn - 1) / bn;
  return (int)((tiles + 15) / 16 * 16);
}
size_t tmax_bytes(const Shape& s) {
  return align_up((size_t)s.B * s.Hq * s.Tq * (size_t)tmax_stride(s) * 2, 256);
}
size_t redo_bytes(const Shape& s) { return align_up(select_chunk_rows(s) * 4, 256); }

// Workspace of hs_full_attn_topk: tile maxima, candidate buffers and row flags when fused,
// else what the larger of its two passes needs.
size_t fused_tokens_ws(const Shape& s, int k_global) {
  if (fused_tokens(s, k_global)) return tmax_bytes(s) + tk_prefill_ws(s) + redo_bytes(s);
  const size_t a = full_attn_ws(s);
  const size_t b = token_select_ws(s, k_global);
  if (b == 0 && token_route(s, k_global) == SEL_NONE) return 0;
  return a > b ? a : b;
}

hs::BlockTopkParams bk_params(const Shape& s, const BkGeom& g, const float* lse, int block,
                              int n_blocks, int32_t* blk_idx, int32_t* count, void* ws) {
  hs::BlockTopkParams p;
  memset(&p, 0, sizeof(p));
  p.lse = lse;
  p.B = s.B;
  p.Tq = s.Tq;
  p.Tk = s.Tk;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = s.g;
  p.q_off = s.q_off;
  p.block = block;
  p.n_blocks = n_blocks;
  p.q_per_set = g.q_per_set;
  p.sets_per_bu = g.sets_per_bu;
  p.n_split = g.n_split;
  p.blocks_per_split = g.blocks_per_split;
  p.scale_log2 = s.scale_log2;
  p.cand = (unsigned long long*)ws;
  p.blk_idx = blk_idx;
  p.cnt = count;
  return p;
}

}  // namespace

extern "C" {

const char* hs_version(void) { return "hysparse-gfx950 0.1"; }

const char* hs_last_error(void) { return g_err; }

const char* hs_status_string(hs_status s) {
  switch (s) {
    case HS_OK: return "ok";
    case HS_ERR_INVALID_ARG: return "invalid argument";
    case HS_ERR_UNSUPPORTED: return "unsupported configuration";
    case HS_ERR_WORKSPACE: return "workspace too small";
    case HS_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t hs_workspace_size(hs_op op, const hs_attn_desc* desc, int32_t p0, int32_t p1) {
  Shape s;
  if (check_desc(desc, &s) != HS_OK) return 0;
  switch (op) {
    case HS_OP_FULL_ATTN: return full_attn_ws(s);
    case HS_OP_ORACLE_TOPK: return token_select_ws(s, p0);
    case HS_OP_FULL_ATTN_TOPK: return fused_tokens_ws(s, p0);
    case HS_OP_BLOCK_TOPK: {
      BkGeom g;
      SelRoute r;
      if (block_route(s, p0, p1, &r, &g) != HS_OK) return 0;
      return block_select_ws(r, s, g, p1);
    }
    case HS_OP_SPARSE_ATTN: {
      if (p0 < 1 || p1 < 0) return 0;
      // the paged call (row kernel) and the contiguous one (group kernel for groups of more
      // than 16 heads) share this size
      const size_t a = sparse_ws(s, sparse_geom(s, p0, p1, false), p1);
      const size_t b = sparse_ws(s, sparse_geom(s, p0, p1, true), p1);
      return a > b ? a : b;
    }
    case HS_OP_FULL_ATTN_LOGITS: return row_fa_ws(s, 0);
    case HS_OP_FULL_ATTN_PAGED: {
      if (p0 < 1 || (p0 & (p0 - 1))) {
        fail(HS_ERR_INVALID_ARG, "page_size %d: must be a power of two", p0);
        return 0;
      }
      if (p1 != 0 && p1 != 1) {
        fail(HS_ERR_INVALID_ARG, "p1 %d: 1 when the call keeps the logits, else 0", p1);
        return 0;
      }
      // the tiled prefill kernel needs none; the row kernel its split partials
      return paged_prefill_attn(s, p1 == 1, p0) ? 0 : row_fa_ws(s, p0);
    }
    case HS_OP_TOPK_FROM_LOGITS: return tk_ws(s, tl_geom(s));
    case HS_OP_FULL_ATTN_BLOCK_TOPK: return fused_blocks_ws(s, p0, p1);
    case HS_OP_BLOCK_TOPK_FROM_LOGITS: {
      BkGeom g;
      if (bk_check(s, p0, p1, &g, true) != HS_OK) return 0;
      return bk_ws(g, p1);
    }
  }
  fail(HS_ERR_INVALID_ARG, "unknown op %d", (int)op);
  return 0;
}

hs_status hs_full_attn_fwd(const hs_attn_desc* desc, const void* q, const void* k, const void* v,
                           void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (!q || !k || !v || !o || !lse) return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (use_prefill_kernel(s)) {
    const hs::PrefillParams pp = prefill_params(s, q, k, v, o, lse);
    return hip_status(hs::launch_prefill_attn(pp, s.D, (hipStream_t)stream), "prefill attention kernel");
  }
  return row_full_attn(s, q, k, v, o, lse, nullptr, ws, ws_bytes, stream);
}

hs_status hs_full_attn_block_topk(const hs_attn_desc* desc, const void* q, const void* k,
                                  const void* v, int32_t block, int32_t n_blocks, void* o,
                                  float* lse, int32_t* blk_idx, int32_t* count, void* ws,
                                  size_t ws_bytes, void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (!q || !k || !v || !o || !lse || !blk_idx || !count)
    return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (fused_blocks(s, block, n_blocks)) {
    hs::PrefillParams pp = prefill_params(s, q, k, v, o, lse);
    pp.blk_idx = blk_idx;
    pp.blk_cnt = count;
    pp.n_blocks = n_blocks;
    return hip_status(hs::launch_prefill_attn(pp, s.D, (hipStream_t)stream),
                      "prefill attention kernel with block selection");
  }
  // two passes: every argument of both is checked before the first launch
  BkGeom g;
  SelRoute r;
  st = block_route(s, block, n_blocks, &r, &g);
  if (st != HS_OK) return st;
  const size_t need = fused_blocks_ws(s, block, n_blocks);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  st = hs_full_attn_fwd(desc, q, k, v, o, lse, ws, ws_bytes, stream);
  if (st != HS_OK) return st;
  return hs_block_score_topk(desc, q, k, lse, block, n_blocks, blk_idx, count, ws, ws_bytes,
                             stream);
}

hs_status hs_full_attn_topk(const hs_attn_desc* desc, const void* q, const void* k, const void* v,
                            int32_t k_global, int32_t window, float bound_margin, void* o,
                            float* lse, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                            void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (!q || !k || !v || !o || !lse || !idx || !count)
    return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (k_global < 0 || window < 0) return fail(HS_ERR_INVALID_ARG, "k_global and window must be >= 0");
  if ((long long)k_global + window < 1) return fail(HS_ERR_INVALID_ARG, "k_global + window must be >= 1");
  if (!finite_bits(bound_margin)) return fail(HS_ERR_INVALID_ARG, "bound_margin must be finite");
  if (token_route(s, k_global) == SEL_NONE)
    return fail(HS_ERR_UNSUPPORTED, "token selection: no route for this shape");
  const size_t need = fused_tokens_ws(s, k_global);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!fused_tokens(s, k_global)) {
    st = hs_full_attn_fwd(desc, q, k, v, o, lse, ws, ws_bytes, stream);
    if (st != HS_OK) return st;
    return hs_oracle_topk(desc, q, k, lse, k_global, window, idx, count, ws, ws_bytes, stream);
  }
  hipStream_t hst = (hipStream_t)stream;
  char* w = (char*)ws;
  uint16_t* tmax = (uint16_t*)w;
  unsigned long long* tbuf = (unsigned long long*)(w + tmax_bytes(s));
  int32_t* redo = (int32_t*)(w + tmax_bytes(s) + tk_prefill_ws(s));
  hs::PrefillParams pp = prefill_params(s, q, k, v, o, lse);
  pp.tile_max = tmax;
  pp.tmax_stride = tmax_stride(s);
  hipError_t e = hs::launch_prefill_attn(pp, s.D, hst);
  if (e != hipSuccess) return hip_status(e, "prefill attention kernel with tile maxima");
  hs::PrefillSelectParams p = select_params(s, q, k, lse);
  p.k_global = k_global;
  p.window = window;
  p.cap = k_global + window;
  p.tbuf = tbuf;
  p.idx = idx;
  p.cnt = count;
  p.tile_max = tmax;
  p.tmax_stride = pp.tmax_stride;
  p.tmax_tile = hs::prefill_tile_keys(s.D);
  p.bound_margin = bound_margin;
  p.redo = redo;
  if (p.chunks > 1)
    p.ccnt = (int32_t*)((char*)tbuf + align_up(select_chunk_rows(s) * hs::prefill_select_buffer_cap() * 8, 256));
  e = hs::launch_prefill_select(p, s.D, false, false, hst);
  if (e != hipSuccess) return hip_status(e, "token selection kernel from the tile-maximum bound");
  // rows whose bound was above their k-th score, selected again without it
  hs::PrefillSelectParams p2 = p;
  p2.tile_max = nullptr;
  p2.redo = nullptr;
  p2.redo_only = redo;
  return hip_status(hs::launch_prefill_select(p2, s.D, false, false, hst),
                    "token selection kernel (second pass)");
}

hs_status hs_full_attn_fwd_logits(const hs_attn_desc* desc, const void* q, const void* k,
                                  const void* v, void* o, float* lse, float* logits, void* ws,
                                  size_t ws_bytes, void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (!q || !k || !v || !o || !lse || !logits) return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  if ((uintptr_t)logits % 4) return fail(HS_ERR_INVALID_ARG, "logits must be 4-byte aligned");
  return row_full_attn(s, q, k, v, o, lse, logits, ws, ws_bytes, stream);
}

hs_status hs_full_attn_fwd_paged(const hs_attn_desc* desc, const void* q, const void* k_pool,
                                 const void* v_pool, const hs_kv_pages* pages, void* o, float* lse,
                                 float* logits, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (!q || !k_pool || !v_pool || !o || !lse) return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  st = check_pages(s, pages);
  if (st != HS_OK) return st;
  if (logits && (uintptr_t)logits % 4) return fail(HS_ERR_INVALID_ARG, "logits must be 4-byte aligned");
  if (paged_prefill_attn(s, logits != nullptr, pages->page_size)) {
    hs::PrefillParams pp = prefill_params(s, q, k_pool, v_pool, o, lse);
    pp.pages = pages->block_table;
    pp.page_shift = __builtin_ctz((unsigned)pages->page_size);
    pp.max_pages = pages->max_pages;
    pp.n_pages = pages->n_pages;
    return hip_status(hs::launch_prefill_attn(pp, s.D, (hipStream_t)stream),
                      "paged prefill attention kernel");
  }
  return row_full_attn(s, q, k_pool, v_pool, o, lse, logits, ws, ws_bytes, stream, pages);
}

hs_status hs_oracle_topk_from_logits(const hs_attn_desc* desc, const float* logits,
                                     const float* lse, int32_t k_global, int32_t window,
                                     int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                                     void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  if (!logits || !lse || !idx || !count) return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (k_global < 0 || window < 0) return fail(HS_ERR_INVALID_ARG, "k_global and window must be >= 0");
  if ((long long)k_global + window < 1) return fail(HS_ERR_INVALID_ARG, "k_global + window must be >= 1");
  const TkGeom t = tl_geom(s);
  const size_t need = tk_ws(s, t);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hs::TopkDecodeParams p = tk_params(s, t, lse, k_global, window, idx, count, ws);
  p.logits = logits;
  return hip_status(hs::launch_topk_from_logits(p, (hipStream_t)stream), "token top-k kernels");
}

hs_status hs_block_topk_from_logits(const hs_attn_desc* desc, const float* logits,
                                    const float* lse, int32_t block, int32_t n_blocks,
                                    int32_t* blk_idx, int32_t* count, void* ws, size_t ws_bytes,
                                    void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  if (!logits || !lse || !blk_idx || !count) return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  BkGeom g;
  st = bk_check(s, block, n_blocks, &g, true);
  if (st != HS_OK) return st;
  const size_t need = bk_ws(g, n_blocks);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hs::BlockTopkParams p = bk_params(s, g, lse, block, n_blocks, blk_idx, count, ws);
  p.logits = logits;
  return hip_status(hs::launch_block_from_logits(p, (hipStream_t)stream), "block top-k kernels");
}


namespace {

// The paged selection calls take the streamed prefill route only (the decode-shaped routes
// select from logits that full attention keeps, which never read the pages), on pages that
// hold whole 64-key tiles.
hs_status check_paged_select(const Shape& s, const hs_kv_pages* pages, SelRoute route) {
  hs_status st = check_pages(s, pages);
  if (st != HS_OK) return st;
  if (pages->page_size < kPagedSelectMinPage)
    return fail(HS_ERR_UNSUPPORTED, "paged selection: page_size %d below %d (pages must hold "
                "whole 64-key tiles)", pages->page_size, kPagedSelectMinPage);
  if (route != SEL_PREFILL)
    return fail(HS_ERR_UNSUPPORTED, "paged selection takes prefill shapes (many query rows per "
                "KV head); for decode keep the logits (hs_full_attn_fwd_paged with logits) and "
                "select from them");
  return HS_OK;
}

void set_select_pages(hs::PrefillSelectParams& p, const hs_kv_pages* pages) {
  if (!pages) return;
  p.pages = pages->block_table;
  p.page_shift = __builtin_ctz((unsigned)pages->page_size);
  p.max_pages = pages->max_pages;
  p.n_pages = pages->n_pages;
}

hs_status token_select(const hs_attn_desc* desc, const void* q, const void* k,
                       const hs_kv_pages* pages, const float* lse, int32_t k_global,
                       int32_t window, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                       void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (!q || !k || !lse || !idx || !count) return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (k_global < 0 || window < 0) return fail(HS_ERR_INVALID_ARG, "k_global and window must be >= 0");
  if ((long long)k_global + window < 1) return fail(HS_ERR_INVALID_ARG, "k_global + window must be >= 1");
  const SelRoute route = token_route(s, k_global);
  if (pages) {
    st = check_paged_select(s, pages, route);
    if (st != HS_OK) return st;
  }
  hipStream_t hst = (hipStream_t)stream;
  if (route == SEL_PREFILL) {
    const size_t need = tk_prefill_ws(s);
    if (!ws || ws_bytes < need)
      return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    hs::PrefillSelectParams p = select_params(s, q, k, lse);
    p.k_global = k_global;
    p.window = window;
    p.cap = k_global + window;
    p.tbuf = (unsigned long long*)ws;
    if (p.chunks > 1)
      p.ccnt = (int32_t*)((char*)ws + align_up(select_chunk_rows(s) * hs::prefill_select_buffer_cap() * 8, 256));
    p.idx = idx;
    p.cnt = count;
    set_select_pages(p, pages);
    return hip_status(hs::launch_prefill_select(p, s.D, s.in_f32, false, hst),
                      "token selection kernel");
  }
  if (route == SEL_DECODE) {
    const TkGeom t = tk_geom(s);
    const size_t need = tk_ws(s, t);
    if (!ws || ws_bytes < need)
      return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    hs::TopkDecodeParams p = tk_params(s, t, lse, k_global, window, idx, count, ws);
    p.q = q;
    p.k = k;
    return hip_status(hs::launch_topk_decode(p, s.D, s.in_f32, hst), "token top-k kernels");
  }
  if (route == SEL_NONE)
    return fail(HS_ERR_UNSUPPORTED, "token selection: %zu bytes of logits for this shape exceed "
                "the %zu-byte bound of the route for this group and head size", logit_bytes(s),
                kMaxLogitBytes);
  // logits of the rows first, then the selection from them
  const TkGeom t = tl_geom(s);
  const size_t lb = logit_bytes(s);
  const size_t need = lb + tk_ws(s, t);
  if (!ws || ws_bytes < need)
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  float* logits = (float*)ws;
  hipError_t e = hs::launch_logits(logits_params(s, q, k, logits), s.D, s.in_f32, hst);
  if (e != hipSuccess) return hip_status(e, "logits kernel");
  hs::TopkDecodeParams p = tk_params(s, t, lse, k_global, window, idx, count, (char*)ws + lb);
  p.logits = logits;
  return hip_status(hs::launch_topk_from_logits(p, hst), "token top-k kernels");
}

hs_status block_select(const hs_attn_desc* desc, const void* q, const void* k,
                       const hs_kv_pages* pages, const float* lse, int32_t block,
                       int32_t n_blocks, int32_t* blk_idx, int32_t* count, void* ws,
                       size_t ws_bytes, void* stream) {
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (!q || !k || !lse || !blk_idx || !count) return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  BkGeom g;
  SelRoute route;
  st = block_route(s, block, n_blocks, &route, &g);
  if (st != HS_OK) return st;
  if (pages) {
    st = check_paged_select(s, pages, route);
    if (st != HS_OK) return st;
  }
  hipStream_t hst = (hipStream_t)stream;
  const size_t need = block_select_ws(route, s, g, n_blocks);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (route == SEL_PREFILL) {
    hs::PrefillSelectParams p = select_params(s, q, k, lse);
    p.block = block;
    p.n_blocks = n_blocks;
    p.idx = blk_idx;
    p.cnt = count;
    if (p.chunks > 1) {
      p.cvals = (unsigned long long*)ws;
      p.ccnt = (int32_t*)((char*)ws + align_up(select_chunk_rows(s) * (size_t)n_blocks * 8, 256));
    }
    set_select_pages(p, pages);
    return hip_status(hs::launch_prefill_select(p, s.D, s.in_f32, true, hst),
                      "block selection kernel");
  }
  if (route == SEL_DECODE) {
    hs::BlockTopkParams p = bk_params(s, g, lse, block, n_blocks, blk_idx, count, ws);
    p.q = q;
    p.k = k;
    return hip_status(hs::launch_block_topk(p, s.D, s.in_f32, hst), "block top-k kernels");
  }
  // logits of the rows first, then the selection from them
  const size_t lb = logit_bytes(s);
  float* logits = (float*)ws;
  hipError_t e = hs::launch_logits(logits_params(s, q, k, logits), s.D, s.in_f32, hst);
  if (e != hipSuccess) return hip_status(e, "logits kernel");
  hs::BlockTopkParams p = bk_params(s, g, lse, block, n_blocks, blk_idx, count, (char*)ws + lb);
  p.logits = logits;
  return hip_status(hs::launch_block_from_logits(p, hst), "block top-k kernels");
}

}  // namespace

hs_status hs_oracle_topk(const hs_attn_desc* desc, const void* q, const void* k, const float* lse,
                         int32_t k_global, int32_t window, int32_t* idx, int32_t* count, void* ws,
                         size_t ws_bytes, void* stream) {
  return token_select(desc, q, k, nullptr, lse, k_global, window, idx, count, ws, ws_bytes,
                      stream);
}

hs_status hs_oracle_topk_paged(const hs_attn_desc* desc, const void* q, const void* k_pool,
                               const hs_kv_pages* pages, const float* lse, int32_t k_global,
                               int32_t window, int32_t* idx, int32_t* count, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!pages) return fail(HS_ERR_INVALID_ARG, "NULL page table");
  return token_select(desc, q, k_pool, pages, lse, k_global, window, idx, count, ws, ws_bytes,
                      stream);
}

hs_status hs_block_score_topk(const hs_attn_desc* desc, const void* q, const void* k,
                              const float* lse, int32_t block, int32_t n_blocks,
                              int32_t* blk_idx, int32_t* count, void* ws, size_t ws_bytes,
                              void* stream) {
  return block_select(desc, q, k, nullptr, lse, block, n_blocks, blk_idx, count, ws, ws_bytes,
                      stream);
}

hs_status hs_block_score_topk_paged(const hs_attn_desc* desc, const void* q, const void* k_pool,
                                    const hs_kv_pages* pages, const float* lse, int32_t block,
                                    int32_t n_blocks, int32_t* blk_idx, int32_t* count, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!pages) return fail(HS_ERR_INVALID_ARG, "NULL page table");
  return block_select(desc, q, k_pool, pages, lse, block, n_blocks, blk_idx, count, ws, ws_bytes,
                      stream);
}

hs_status hs_sparse_attn_gather(const hs_attn_desc* desc, const void* q, const void* k_full,
                                const void* v_full, hs_index_kind kind, const int32_t* idx,
                                const int32_t* count, int32_t idx_cap, int32_t block,
                                const hs_swa_branch* swa, void* o, float* lse_opt, void* ws,
                                size_t ws_bytes, void* stream) {
  return hs_sparse_attn_gather_ex(desc, q, k_full, v_full, kind, idx, count, idx_cap, block, swa,
                                  nullptr, o, lse_opt, ws, ws_bytes, stream);
}

hs_status hs_sparse_attn_gather_ex(const hs_attn_desc* desc, const void* q, const void* k_full,
                                   const void* v_full, hs_index_kind kind, const int32_t* idx,
                                   const int32_t* count, int32_t idx_cap, int32_t block,
                                   const hs_swa_branch* swa, const hs_sparse_opts* opts, void* o,
                                   float* lse_opt, void* ws, size_t ws_bytes, void* stream) {
  return hs_sparse_attn_gather_paged(desc, q, k_full, v_full, nullptr, kind, idx, count, idx_cap,
                                     block, swa, opts, o, lse_opt, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Body of every sparse-layer entry point.  from_scratch: the workspace is the library's
// device-resident scratch (the no-allocation entry point), fetched after validation.
hs_status sparse_layer(const hs_attn_desc* desc, const void* q, const void* k_full,
                       const void* v_full, const hs_kv_pages* pages, hs_index_kind kind,
                       const int32_t* idx, const int32_t* count, int32_t idx_cap, int32_t block,
                       const hs_swa_branch* swa, const hs_sparse_opts* opts, void* o,
                       float* lse_opt, void* ws, size_t ws_bytes, void* stream,
                       bool from_scratch) {
  const float* sink_g = opts ? opts->sink : nullptr;
  const float* sink_l = opts ? opts->sink_local : nullptr;
  const float* ogate = opts ? opts->out_gate : nullptr;
  const int ring = opts ? opts->local_ring : 0;
  const int gate_ch = opts ? opts->gates_per_channel : 0;
  Shape s;
  hs_status st = check_desc(desc, &s);
  if (st != HS_OK) return st;
  st = check_qkv_dtype(s);
  if (st != HS_OK) return st;
  if (pages) {
    st = check_pages(s, pages);
    if (st != HS_OK) return st;
  }
  if (!q || !k_full || !v_full || !idx || !count || !o)
    return fail(HS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (kind != HS_IDX_TOKEN && kind != HS_IDX_BLOCK) return fail(HS_ERR_INVALID_ARG, "unknown index kind");
  if (idx_cap < 1) return fail(HS_ERR_INVALID_ARG, "idx_cap must be >= 1");
  if (kind == HS_IDX_BLOCK && block < 1) return fail(HS_ERR_INVALID_ARG, "block must be >= 1");
  const long long keys = kind == HS_IDX_TOKEN ? idx_cap : (long long)idx_cap * block;
  if (keys > (1LL << 30)) return fail(HS_ERR_UNSUPPORTED, "index set too large");
  int window = 0;
  if (swa) {
    if (!swa->k_local || !swa->v_local || !swa->gate_logits)
      return fail(HS_ERR_INVALID_ARG, "NULL pointer in the sliding-window branch");
    if (swa->window < 1) return fail(HS_ERR_INVALID_ARG, "sliding window must be >= 1");
    window = swa->window;
  }
  if (sink_l && !swa)
    return fail(HS_ERR_INVALID_ARG, "sink_local given without a sliding-window branch");
  if (gate_ch != 0 && gate_ch != 1)
    return fail(HS_ERR_INVALID_ARG, "gates_per_channel must be 0 or 1, got %d", gate_ch);
  if (ring < 0 || (ring > 0 && !swa))
    return fail(HS_ERR_INVALID_ARG, "local_ring %d: needs a sliding-window branch", ring);
  // the q_len rows of one call read positions q_offset - window + 1 .. q_offset + q_len - 1,
  // which must sit in distinct ring slots
  if (ring > 0 && (long long)ring < (long long)window + s.Tq - 1)
    return fail(HS_ERR_INVALID_ARG,
                "local_ring %d shorter than window + q_len - 1 = %lld (window %d, q_len %d)",
                ring, (long long)window + s.Tq - 1, window, s.Tq);
  const SparseGeom g = sparse_geom(s, keys, window, pages != nullptr);
  const size_t need = sparse_ws(s, g, window);
  if (from_scratch) {
    if (need > hs::kScratchBytes)
      return fail(HS_ERR_WORKSPACE,
                  "this layer needs %zu bytes of split partials; the no-allocation entry point "
                  "holds at most %zu (use hs_sparse_attn_gather with a workspace)",
                  need, hs::kScratchBytes);
    hipError_t e = hs::scratch_buffer(&ws);
    if (e != hipSuccess) return hip_status(e, "device scratch of the no-allocation entry point");
    ws_bytes = hs::kScratchBytes;
  }
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(HS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hipStream_t hst = (hipStream_t)stream;

  hs::RowAttnParams pg = ra_params(s, g.glob);
  pg.q = q;
  pg.k = k_full;
  pg.v = v_full;
  pg.idx = idx;
  pg.cnt = count;
  pg.idx_cap = idx_cap;
  pg.block = block;
  pg.o = o;
  pg.lse = lse_opt;
  pg.final_direct = !g.combine;
  pg.sink = sink_g;
  pg.sink2 = sink_l;
  pg.out_gate = ogate;
  pg.gate_ch = gate_ch;
  pg.ring = ring;
  pg.query_major = g.glob.sets_per_bu > 1;  // many queries: one (b, u)'s rows at a time
  if (pages) set_pages(pg, pages);
  const hs::KeySrc src = kind == HS_IDX_TOKEN ? hs::SRC_TOKEN : hs::SRC_BLOCK;
  if (g.fused) {
    pg.k2 = swa->k_local;
    pg.v2 = swa->v_local;
    pg.window = window;
    pg.gate = swa->gate_logits;
    hipError_t e = hs::launch_row_attn(pg, s.D, s.in_f32, src, hst, true, g.wide);
    if (e != hipSuccess) return hip_status(e, "gated sparse attention kernel");
    return ok();
  }
  char* w = (char*)ws;
  if (g.combine) {
    carve_partials(w, g.glob, s.D, &pg.part_m, &pg.part_l, &pg.part_o);
    w += partial_bytes(g.glob, s.D);
  }
  hs::RowAttnParams pl;
  if (window > 0) {
    pl = ra_params(s, g.loc);
    pl.q = q;
    pl.k = swa->k_local;
    pl.v = swa->v_local;
    pl.window = window;
    pl.ring = ring;
    pl.final_direct = 0;
    carve_partials(w, g.loc, s.D, &pl.part_m, &pl.part_l, &pl.part_o);
  }
  hipError_t e;
  if (window > 0 && !g.group && !g.wide) {  // both branches in one launch
    e = hs::launch_row_attn_two(pg, pl, s.D, s.in_f32, src, hst);
    if (e != hipSuccess) return hip_status(e, "sparse attention kernel (two branches)");
  } else {
    e = g.group ? hs::launch_group_attn(pg, s.D, src, hst)
                : hs::launch_row_attn(pg, s.D, s.in_f32, src, hst, false, g.wide);
    if (e != hipSuccess) return hip_status(e, "sparse attention kernel");
    if (window > 0) {
      e = hs::launch_row_attn(pl, s.D, s.in_f32, hs::SRC_WINDOW, hst);
      if (e != hipSuccess) return hip_status(e, "sliding-window kernel");
    }
  }
  if (g.combine) {
    hs::CombineParams c = combine_params(s, g.glob, o, lse_opt);
    c.n_branch = window > 0 ? 2 : 1;
    c.sink[0] = sink_g;
    c.sink[1] = sink_l;
    c.out_gate = ogate;
    c.gate_ch = gate_ch;
    c.m[0] = pg.part_m;
    c.l[0] = pg.part_l;
    c.po[0] = pg.part_o;
    c.n_split[0] = g.glob.n_split;
    if (window > 0) {
      c.m[1] = pl.part_m;
      c.l[1] = pl.part_l;
      c.po[1] = pl.part_o;
      c.n_split[1] = g.loc.n_split;
      c.gate = swa->gate_logits;
    }
    e = hs::launch_combine(c, s.D, hst);
    if (e != hipSuccess) return hip_status(e, "combine kernel");
  }
  return ok();
}

}  // namespace

extern "C" {

hs_status hs_sparse_attn_gather_paged(const hs_attn_desc* desc, const void* q, const void* k_full,
                                      const void* v_full, const hs_kv_pages* pages,
                                      hs_index_kind kind, const int32_t* idx,
                                      const int32_t* count, int32_t idx_cap, int32_t block,
                                      const hs_swa_branch* swa, const hs_sparse_opts* opts,
                                      void* o, float* lse_opt, void* ws, size_t ws_bytes,
                                      void* stream) {
  return sparse_layer(desc, q, k_full, v_full, pages, kind, idx, count, idx_cap, block, swa, opts,
                      o, lse_opt, ws, ws_bytes, stream, false);
}

hs_status hs_sparse_attn_gather_noalloc(const hs_attn_desc* desc, const void* q,
                                        const void* k_full, const void* v_full,
                                        hs_index_kind kind, const int32_t* idx,
                                        const int32_t* count, int32_t idx_cap, int32_t block,
                                        const hs_swa_branch* swa, void* o, float* lse_opt,
                                        void* stream) {
  return sparse_layer(desc, q, k_full, v_full, nullptr, kind, idx, count, idx_cap, block, swa,
                      nullptr, o, lse_opt, nullptr, 0, stream, true);
}

}  // extern "C"
