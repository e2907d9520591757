// hs_kernels.h -- launch interface between the C ABI layer (abi.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

// Where the keys of one row-set come from.
enum KeySrc : int {
  SRC_RANGE = 0,  // contiguous positions lo..hi (full attention, sliding window)
  SRC_TOKEN = 1,  // token positions from an index list
  SRC_BLOCK = 2,  // whole blocks of `block` positions from a block-id list
  SRC_WINDOW = 3  // contiguous positions t-window+1 .. t (sliding window over own K', V')
};

// One launch of the row-attention kernel.  A row-set is a group of at most 16 (query, head)
// rows that share one KV head and one key list; its rows are packed in the MFMA M dimension.
struct RowAttnParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;  // list modes: [B, Tq, Hkv, idx_cap]
  const int32_t* cnt;  // list modes: [B, Tq, Hkv]
  int idx_cap, block;
  int window;  // window mode: each row sees positions t-window+1 .. t
  int B, Tq, Tk, Hq, Hkv, g;
  int hpc, cpq;     // heads per row-set (min(g, 16)) and head chunks per query (g / hpc)
  long long q_off;
  int q_per_set;    // queries per row-set (range mode may pack several; list modes: 1)
  int sets_per_bu;  // row-sets per (b, u) = ceil(Tq / q_per_set)
  int n_split;      // splits of the key list per row-set (grid.x)
  int steps_per_split;  // 32-key steps per split
  float scale_log2;     // log2(e) / sqrt(d)
  // final output (when final_direct) or partials (otherwise)
  void* o;
  float* lse;
  int out_f32;
  int final_direct;
  float* part_m;   // [n_split][n_sets][16]
  double* part_l;  // [n_split][n_sets][16]
  float* part_o;   // [n_split][n_sets][16][D]
  // gated layer in one pass (no splits): the window branch's own K', V' and the gate logits
  const void* k2;
  const void* v2;
  const float* gate;  // [B, Tq, Hq, 2]
  // full attention (range mode, 4 waves) may also store its raw dot products q.k:
  float* logits;   // [B, Tq, Hq, Tk] fp32, or null
  int logits_vec;  // 16-byte stores allowed (Tk % 4 == 0 and an aligned base)
  // optional per-head sink logits (sink: this pass; sink2: the window branch of the gated
  // one-pass layer) and sigmoid output-gate logits, applied when the output is final
  const float* sink;      // [Hq] or null
  const float* sink2;     // [Hq] or null
  const float* out_gate;  // [B, Tq, Hq] or null
  int gate_ch;  // gates per channel: gate [B, Tq, Hq, 2, D], out_gate [B, Tq, Hq, D]
  // paged K / V (range and list sources): pools [n_pages, page_size, Hkv, d], page of logical
  // page lp of batch entry b = pages[b * max_pages + lp]; page_size a power of two
  const int32_t* pages;
  int page_size, max_pages, n_pages;
  int ring;  // window source: K2 / V2 (or K / V) are rings [B, ring, Hkv, d], slot t % ring (0: none)
  int query_major;  // workgroup order: query fastest (else KV head fastest)
};

// Merge of split partials (one or two branches) into O and LSE; with two branches the sigmoid
// gates combine them.
struct CombineParams {
  const float* m[2];
  const double* l[2];
  const float* po[2];
  int n_split[2];
  int n_branch;
  const float* gate;  // [B, Tq, Hq, 2] (two branches)
  int B, Tq, Hq, Hkv, g;
  int hpc, cpq;
  int q_per_set, sets_per_bu;
  void* o;
  float* lse;  // nullable; LSE of branch 0
  int out_f32;
  const float* sink[2];   // per branch: [Hq] sink logits or null
  const float* out_gate;  // [B, Tq, Hq] sigmoid output-gate logits or null
  int gate_ch;  // gates per channel: gate [B, Tq, Hq, 2, D], out_gate [B, Tq, Hq, D]
};

// gated: list source (token or block) then the window branch over k2, v2 in one workgroup,
// combined with the sigmoid gates (requires n_split == 1).  wide: 8 waves per workgroup instead
// of 4 (bf16 only), for unsplit key lists of few row-sets.
hipError_t launch_row_attn(const RowAttnParams& p, int head_dim, bool in_f32, KeySrc src,
                           hipStream_t stream, bool gated = false, bool wide = false);
// Both branches of a gated layer whose lists are split, in one launch of 4-wave workgroups: the
// token / block lists of pg (src), then the sliding window of pl (window source, not paged); both
// write split partials.
hipError_t launch_row_attn_two(const RowAttnParams& pg, const RowAttnParams& pl, int head_dim,
                               bool in_f32, KeySrc src, hipStream_t stream);

// Attention for groups of 32, 48 or 64 heads (bf16, head_dim 128 or 256) over a range (full
// attention, optional logits as in the row kernel) or a token / block list (steps_per_split 64-key
// steps of at most 2048 entries): one workgroup per (batch entry, KV head, query, split), one
// wave per 16-head chunk, K / V steps shared through LDS; always writes split partials (hpc 16,
// q_per_set 1, sets_per_bu Tq).  List offsets are 32-bit: Tk * Hkv * d * 2 below 2^31.
hipError_t launch_group_attn(const RowAttnParams& p, int head_dim, KeySrc src, hipStream_t stream);

// Full causal attention for many queries per KV head (bf16): 256 (query, head) rows per
// workgroup sharing LDS-staged K/V tiles.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  int B, Tq, Tk, Hq, Hkv, g;
  long long q_off;
  float scale_log2;
  void* o;
  float* lse;
  int out_f32;
  // block selection in the same pass (blocks of 64 keys, n_blocks <= 16), or null
  int32_t* blk_idx;  // [B, Tq, Hkv, n_blocks]
  int32_t* blk_cnt;  // [B, Tq, Hkv]
  int n_blocks;
  // or null: every row's raw logit maximum over each key tile (prefill_tile_keys(head_dim)
  // keys), as bf16 bits rounded toward -inf, [B, Hq, Tq, tmax_stride] (tmax_stride a multiple of
  // 16 and >= the tiles of the row)
  uint16_t* tile_max;
  int tmax_stride;
  // or null: k, v are page pools [n_pages, 1 << page_shift, Hkv, D] and position i of batch
  // entry b lives in page pages[b * max_pages + (i >> page_shift)]; pages hold whole key tiles
  // (1 << page_shift >= prefill_tile_keys(head_dim)), so a tile is one contiguous run of rows
  const int32_t* pages;
  int page_shift, max_pages, n_pages;
};
int prefill_tile_keys(int head_dim);
hipError_t launch_prefill_attn(const PrefillParams& p, int head_dim, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, int head_dim, hipStream_t stream);

// ---- token top-k for row groups of at most 16 (query, head) rows (decode) ----------------
struct TopkDecodeParams {
  const void* q;
  const void* k;
  const float* lse;
  int B, Tq, Tk, Hq, Hkv, g;
  long long q_off;
  int k_global, window;
  int q_per_set, sets_per_bu;   // query rows packed per score workgroup (q_per_set * g <= 16)
  int n_split, keys_per_split;  // score pass: key chunk per workgroup (multiple of 64)
  int sel_split, keys_per_sel;  // selection passes: key chunk per workgroup
  float scale_log2;
  // workspace
  uint32_t* keys;               // [rows][Tk]   rows = B * Tq * Hkv
  uint32_t* hist;               // [rows][2048] top-11-bit histograms, followed by `bcount`
  uint32_t* bcount;             // [rows] boundary-list lengths
  unsigned long long* blist;    // [rows][Tk] boundary list (key << 32 | ~position)
  uint32_t* above;              // [rows][sel_split] keys above the boundary bin, per chunk
  uint32_t* counts;             // [rows][sel_split] keys taken per chunk
  uint32_t* state;              // [rows][2] key threshold T, last position taken at T
  // outputs
  int32_t* idx;  // [B, Tq, Hkv, cap]
  int32_t* cnt;  // [B, Tq, Hkv]
  int cap;
  // selection from stored logits instead of Q, K (launch_topk_from_logits; n_split chunks of
  // keys_per_split keys per (b, t, u) row, multiples of 1024)
  const float* logits;  // [B, Tq, Hq, Tk] raw dot products q.k
};
hipError_t launch_topk_decode(const TopkDecodeParams& p, int head_dim, bool in_f32,
                              hipStream_t stream);
// Whether rows of Tk keys take the chain of collect / finalize / write over key chunks, which
// needs the boundary list, the per-chunk counts and the threshold state; shorter rows are
// selected by one workgroup per row, which needs only the keys and the histograms.
bool topk_decode_uses_chain(long long Tk);
hipError_t launch_topk_from_logits(const TopkDecodeParams& p, hipStream_t stream);

// ---- block scores + top-n blocks ----------------------------------------------------------
struct BlockTopkParams {
  const void* q;
  const void* k;
  const float* lse;
  int B, Tq, Tk, Hq, Hkv, g;
  long long q_off;
  int block, n_blocks;
  int q_per_set, sets_per_bu;
  int n_split, blocks_per_split;
  float scale_log2;
  unsigned long long* cand;  // workspace [rows][n_split][n_blocks]
  int32_t* blk_idx;          // [B, Tq, Hkv, n_blocks]
  int32_t* cnt;              // [B, Tq, Hkv]
  // selection from stored logits instead of Q, K (launch_block_from_logits; one (b, t, u) row
  // per workgroup and split, at most 256 blocks per split)
  const float* logits;  // [B, Tq, Hq, Tk] raw dot products q.k
};
hipError_t launch_block_topk(const BlockTopkParams& p, int head_dim, bool in_f32,
                             hipStream_t stream);
hipError_t launch_block_from_logits(const BlockTopkParams& p, hipStream_t stream);

// ---- selection for many queries per KV head (prefill), streamed tile by tile -----------------
struct PrefillSelectParams {
  const void* q;
  const void* k;
  const float* lse;
  int B, Tq, Tk, Hq, Hkv, g;
  long long q_off;
  float scale_log2;
  // token mode
  int k_global, window, cap;
  unsigned long long* tbuf;  // workspace [rows][prefill_select_buffer_cap()]
  // block mode
  int block, n_blocks;
  // outputs
  int32_t* idx;
  int32_t* cnt;
  // groups of more than 16 heads: `chunks` chunks of 16 heads select on their own (rows of
  // virtual KV head u * chunks + c), keeping their candidates with their values; a merge over the
  // chunks gives the group's set (exact: a key among the group's best is among the best of the
  // chunk that attains its group maximum).  chunks == 1: the group selects as a whole.
  int chunks;
  int32_t* ccnt;               // [B, Tq, Hkv * chunks] entries kept per chunk row
  unsigned long long* cvals;   // block mode: [B, Tq, Hkv * chunks, n_blocks] kept values
  // token mode, or null: the tile maxima of the full-attention pass (PrefillParams::tile_max),
  // from which every row starts at a proven lower bound of its k-th score minus bound_margin;
  // redo[row] (written for every chunk row) then flags the rows whose bound turned out too high
  const uint16_t* tile_max;
  int tmax_stride, tmax_tile;  // tile maxima per row, keys per tile
  float bound_margin;
  int32_t* redo;
  // or null: only workgroups holding a row flagged here run (the rows' second pass)
  const int32_t* redo_only;
  // or null: k is a page pool [n_pages, 1 << page_shift, Hkv, D] addressed through the block
  // table as in PrefillParams; pages hold whole 64-key tiles (page_shift >= 6)
  const int32_t* pages;
  int page_shift, max_pages, n_pages;
};
int prefill_select_buffer_cap();
int prefill_select_max_k();
hipError_t launch_prefill_select(const PrefillSelectParams& p, int head_dim, bool in_f32,
                                 bool block_mode, hipStream_t stream);

// ---- raw logits of few query rows (selection for shapes outside the fused score passes) ----
struct LogitsParams {
  const void* q;
  const void* k;
  int B, Tq, Tk, Hq, Hkv, g;
  long long q_off;
  int n_split, keys_per_split;  // key chunk per workgroup (a multiple of 256)
  float* logits;                // [B, Tq, Hq, Tk] fp32: entries 0..t of query row t
};
hipError_t launch_logits(const LogitsParams& p, int head_dim, bool in_f32, hipStream_t stream);

// ---- device-resident scratch of the no-allocation sparse-layer entry point ------------------
// kScratchBytes of device memory held by the library for the life of the process, one copy per
// device; scratch_buffer returns the current device's copy (its address is looked up once per
// device).  Calls that use it and overlap on one device race.
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t scratch_buffer(void** ptr);

}  // namespace hs
