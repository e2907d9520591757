/*
 * hysparse.h -- C ABI of the HySparse / HySparse2 attention hot path on MI355X (gfx950).
 *
 * Sources (web pages) cited below:
 *   [P1] "HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing", reading notes,
 *        qqtang-code.github.io.
 *   [P2] "HySparse hybrid sparse attention (part 1): full attention as the oracle",
 *        pinghaoyang.com.cn.
 *   [P4] "HySparse: A Hybrid Sparse Attention Architecture with Oracle Token Selection and KV
 *        Cache Sharing", papercache.org summary of arXiv:2602.03560.
 *   [P5] "HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing", picx.dev summary.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE memory owned by the caller (e.g. torch tensors).  The
 *     library never allocates, frees or synchronizes; every call enqueues its kernels on
 *     `stream` (a hipStream_t, NULL = the default stream) and returns.  Device faults surface at
 *     the caller's next synchronization.
 *   - Layouts are contiguous, head_dim fastest:
 *       Q, Q', O : [B, q_len, Hq, d]        K, V, K', V' : [B, kv_len, Hkv, d]
 *       LSE      : [B, Hq, q_len] fp32 (natural log)
 *     Query row j sits at absolute position t = q_offset + j and sees keys 0..t (causal).
 *     Query head h reads KV head u = h / g, g = Hq / Hkv.
 *   - Arguments are validated on the host before anything is enqueued.  An invalid call returns
 *     HS_ERR_INVALID_ARG or HS_ERR_UNSUPPORTED, enqueues nothing and leaves every output
 *     untouched; hs_last_error() then describes the problem.  A failed launch returns HS_ERR_HIP.
 *   - Outputs are fully overwritten (padding included).  The library keeps no state between
 *     calls: the caller keeps K, V and the index sets alive across the sparse layers that reuse
 *     them [P2 engineering constraint 6: producer/consumer lifetime].
 *   - Workspace: every call takes a caller-owned device scratch buffer of at least
 *     hs_workspace_size(...) bytes (16-byte aligned); a smaller one returns HS_ERR_WORKSPACE.
 *   - Supported: head_dim in {64, 128} (fp32 or bf16 inputs) or 256 (bf16; the HySparse2 head
 *     shape, MQA with 64 query heads of d 256 [P1 section 6.1]); g = Hq/Hkv integral and at
 *     most 64 (groups above 16 heads run as chunks of 16, the last one short when g is not a
 *     multiple of 16; the group shares one index set through the maximum over all its heads,
 *     [P2 "Why GQA shares the index within a group"]); kv_len <= 2^30; out_dtype bf16 or fp32.
 *     Block selection needs block a multiple of 16 and 1 <= n_blocks <= 64.  Index selection
 *     from Q and K takes every such shape: many query rows stream over K tiles (groups of up
 *     to 16 heads padded to 4, 8 or 16; larger groups, given at least 16 queries, in chunks of
 *     16 heads whose candidates are merged exactly); few rows with g in {4, 8, 16} and
 *     head_dim <= 128
 *     run the fused score passes; every other shape first computes the rows' raw logits into
 *     the workspace (at most 8 GiB of them: B * q_len * Hq * kv_len * 4 bytes, else
 *     HS_ERR_UNSUPPORTED) and selects from them like stored logits.  Full attention with many
 *     query rows per KV head runs a tiled kernel (bf16; 256 rows per workgroup, 128 at head
 *     size 256, which the group size must divide); the gated sparse layer at head size 256
 *     runs its two branches as split partials plus a combine.  Anything else returns
 *     HS_ERR_UNSUPPORTED.
 *   - Workspace sizes, for orientation: token selection with many query rows per KV head and
 *     k_global <= 1024 keeps a 16 KiB candidate buffer per (b, t, u); with few rows it keeps
 *     4 bytes per candidate key per (b, t, u) plus an 8 KiB histogram (12 bytes per key past
 *     131072 keys, where a boundary list joins them); split attention keeps
 *     per-split partial rows (about 0.5 KiB each).  Full attention with many query rows and the
 *     prefill-shaped block selection need none.
 */
#ifndef HYSPARSE_H
#define HYSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = -1,
  HS_ERR_UNSUPPORTED = -2,
  HS_ERR_WORKSPACE = -3,
  HS_ERR_HIP = -4
} hs_status;

typedef enum { HS_BF16 = 0, HS_F32 = 1 } hs_dtype;

typedef enum { HS_IDX_TOKEN = 0, HS_IDX_BLOCK = 1 } hs_index_kind;

typedef enum {
  HS_OP_FULL_ATTN = 0,   /* p0, p1 unused */
  HS_OP_ORACLE_TOPK = 1, /* p0 = k_global, p1 = window */
  HS_OP_BLOCK_TOPK = 2,  /* p0 = block, p1 = n_blocks */
  HS_OP_SPARSE_ATTN = 3, /* p0 = number of keys per index set (token cap, or n_blocks*block);
                            p1 = SWA window (0: no SWA branch) */
  HS_OP_FULL_ATTN_LOGITS = 4,       /* p0, p1 unused */
  HS_OP_TOPK_FROM_LOGITS = 5,       /* p0 = k_global, p1 = window */
  HS_OP_BLOCK_TOPK_FROM_LOGITS = 6, /* p0 = block, p1 = n_blocks */
  HS_OP_FULL_ATTN_BLOCK_TOPK = 7,   /* p0 = block, p1 = n_blocks */
  HS_OP_FULL_ATTN_PAGED = 8,        /* p0 = page_size; p1 = 1 when the call keeps the logits,
                                       else 0 (a prefill shape without logits needs none) */
  HS_OP_FULL_ATTN_TOPK = 9          /* p0 = k_global, p1 = window */
} hs_op;

typedef struct {
  int32_t batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim;
  int64_t q_offset;   /* absolute position of query row 0; -1 means kv_len - q_len */
  float scale;        /* logit scale tau in a = tau q.k; 0 means 1/sqrt(head_dim) [P2 attention
                         equations]; finite and >= 0.  The calls of one hybrid block (full layer,
                         selection, sparse layers) must use the same value. */
  hs_dtype in_dtype;  /* element type of Q, K, V (and K', V') */
  hs_dtype out_dtype; /* element type of O */
} hs_attn_desc;

/* Sliding-window branch of a HySparse sparse layer: the layer's own local keys and values and
 * the two gate logits per query head [P2 "Same query, two memories" and "Two sigmoid gates";
 * P4 section 3.3]. */
typedef struct {
  const void* k_local;      /* [B, kv_len, Hkv, d], in_dtype; position-indexed */
  const void* v_local;      /* [B, kv_len, Hkv, d], in_dtype */
  const float* gate_logits; /* [B, q_len, Hq, 2] fp32: (zG, zL); sigmoid applied inside
                               ([B, q_len, Hq, 2, d] with hs_sparse_opts.gates_per_channel) */
  int32_t window;           /* w >= 1: positions max(0, t-w+1) .. t */
} hs_swa_branch;

/* Full causal GQA attention, the full-attention layer of a hybrid block:
 *   a_{t,i} = tau q_t.k_i (tau = desc->scale, by default 1/sqrt(d)),
 *   O_t = sum_{i<=t} softmax_i(a) v_i,  LSE_t = ln sum_{i<=t} e^a
 * [P2 "Extracting block scores from exact attention", attention equations; P4 section 3.2].
 * q, k, v: in_dtype.  o: [B, q_len, Hq, d] out_dtype.  lse: [B, Hq, q_len] fp32, required (the
 * index-selection calls normalize logits with it). */
hs_status hs_full_attn_fwd(const hs_attn_desc* desc, const void* q, const void* k, const void* v,
                           void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Token-level oracle index of HySparse2 [P1 section 4.2 changes 1 and 2; P5 "KV Reuse (Inner
 * Level)"].  Per (b, t, u): score s_i = max over the group's heads h of exp(a^h_{t,i} - LSE^h_t)
 * (the group maximum of [P2 "GQA: the group shares one index set"] applied to tokens); the set is
 * the forced window {max(0,t-w+1)..t} plus the k_global best candidates among 0..t-w ranked by
 * (score desc, position asc).  Exact: no candidate is dropped by an approximation.
 * lse: output of hs_full_attn_fwd.  idx: [B, q_len, Hkv, k_global + window] int32, ascending,
 * padded with -1.  count: [B, q_len, Hkv] int32 = min(t+1, k_global + window). */
hs_status hs_oracle_topk(const hs_attn_desc* desc, const void* q, const void* k, const float* lse,
                         int32_t k_global, int32_t window, int32_t* idx, int32_t* count, void* ws,
                         size_t ws_bytes, void* stream);

/* Block-level oracle index of HySparse [P2 "Extracting block scores from exact attention",
 * block-score and TopK equations; P2 "GQA: the group shares one index set"; P4 section 3.2 and
 * Algorithm 1, with the exponential its block-score normalization omits].  Per (b, t, u): S_r = max over heads h and keys
 * i in [rB, min(rB+B-1, t)] of exp(a^h_{t,i} - LSE^h_t), for the causal blocks r <= t/B; the
 * n_blocks best by (S desc, r asc).  blk_idx: [B, q_len, Hkv, n_blocks] int32 ascending, -1
 * padded; count: [B, q_len, Hkv] = min(n_blocks, t/B + 1). */
hs_status hs_block_score_topk(const hs_attn_desc* desc, const void* q, const void* k,
                              const float* lse, int32_t block, int32_t n_blocks,
                              int32_t* blk_idx, int32_t* count, void* ws, size_t ws_bytes,
                              void* stream);

/* Options of a sparse layer (hs_sparse_attn_gather_ex); a NULL field is left out.
 *   sink, sink_local: per-head sink logits of the global (token or block) branch and of the
 *     sliding-window branch, fp32 [Hq], natural log.  The pages give every sparse and
 *     sliding-window layer a learnable per-head sink bias in the manner of gpt-oss [P1 section
 *     6.1; P4 experimental setup]; the reading taken is gpt-oss's: the sink s_h is one more logit in the
 *     softmax denominator and carries no value, p_i = e^{a_i} / (e^{s_h} + sum_j e^{a_j}).  The
 *     reported LSE includes it.  A row with no key then gets o = 0 and LSE = s_h.
 *   out_gate: logits of the sigmoid output gate of those layers [P1 section 6.1], fp32
 *     [B, q_len, Hq], one per (query, head) (the pages give no size; one scalar per head, like
 *     the branch gates): o <- sigmoid(g) * o, applied last.
 *   gates_per_channel: 0 (default) as above; 1: every gate acts per channel [P2 "Two sigmoid
 *     gates, not one of two": the branch gates may act per head or per channel, combined by an
 *     element-wise product], so swa->gate_logits is [B, q_len, Hq, 2, d] (the d logits of zG,
 *     then the d of zL, for each (query, head)) and out_gate is [B, q_len, Hq, d]:
 *     o_c = sigmoid(out_c) (sigmoid(zG_c) o_glob,c + sigmoid(zL_c) o_loc,c).  Other values:
 *     HS_ERR_INVALID_ARG. */
typedef struct {
  const float* sink;
  const float* sink_local;
  const float* out_gate;
  int32_t local_ring; /* 0: swa->k_local / v_local are position-indexed [B, kv_len, Hkv, d];
                         > 0: they are rings [B, local_ring, Hkv, d] holding position t in slot
                         t % local_ring, with local_ring >= window + q_len - 1 (every position a
                         call's rows read in its own slot; else HS_ERR_INVALID_ARG), the
                         layer's own small cache
                         [P2 "Why the local branch cannot reuse the same KV": each sparse layer
                         keeps its own K', V' only for a ring window of length w] */
  int32_t gates_per_channel;
} hs_sparse_opts;

/* Paged K / V cache (serving): K and V are pools [n_pages, page_size, Hkv, d]; the positions
 * p * page_size .. (p + 1) * page_size - 1 of batch entry b live in the pool's page
 * block_table[b * max_pages + p].  Index sets keep logical positions (token) or logical 64-key
 * blocks, whatever the page size; the kernels translate every key position through the table
 * while they load K / V, so no contiguous copy of the cache is made [P2 engineering constraints
 * 2 and 3: logical blocks may span several physical pages, the block table translates them,
 * and the kernel should consume it directly instead of copying to a temporary buffer].
 * page_size: a power of two; max_pages * page_size >= kv_len.  Table entries outside
 * [0, n_pages) are clamped into the pool (the result is then wrong, the read stays inside it). */
typedef struct {
  const int32_t* block_table; /* [B, max_pages] int32, device memory */
  int32_t page_size;
  int32_t max_pages;
  int32_t n_pages;
} hs_kv_pages;

/* Full attention and block-level oracle index in one call: the outputs of hs_full_attn_fwd
 * (o, lse) and of hs_block_score_topk (blk_idx, count) for the same inputs.  The pages obtain
 * the block scores inside the attention loop, from each tile's row maximum, and normalize them
 * with the LSE at the end [P4 Algorithm 1; P2 "Extracting block scores from exact attention"].
 * For prefill-shaped bf16 calls (the tiled prefill kernel: q_len * g > 16) with block == 64 and
 * n_blocks <= 16 this is one pass: every (query, head) row keeps its best n blocks by raw logit
 * maximum while the key tiles stream past (within one head p ranks like the logit), and the g
 * rows of a query merge their lists once their LSEs are known.  Exact: a block among the
 * group's best n is among the best n of the head attaining its group maximum.  No score matrix
 * and no workspace.  Other shapes run the two calls one after the other (same limits as those;
 * workspace: hs_workspace_size(HS_OP_FULL_ATTN_BLOCK_TOPK, desc, block, n_blocks)).  Index
 * sets equal hs_block_score_topk's except where two blocks' scores tie to within fp32
 * rounding (the logits come from a different MFMA tiling). */
hs_status hs_full_attn_block_topk(const hs_attn_desc* desc, const void* q, const void* k,
                                  const void* v, int32_t block, int32_t n_blocks, void* o,
                                  float* lse, int32_t* blk_idx, int32_t* count, void* ws,
                                  size_t ws_bytes, void* stream);

/* Full attention and token-level oracle index in one call: the outputs of hs_full_attn_fwd
 * (o, lse) and of hs_oracle_topk (idx, count) for the same inputs, the same bit for bit.  For
 * prefill-shaped bf16 calls with head_dim up to 128 (those on the tiled prefill attention kernel
 * and the streamed prefill selection) the attention pass also records every (query, head) row's
 * largest logit in each 64-key tile, and the selection pass starts every (b, t, u) (for groups of
 * more than 16 heads every chunk of 16 heads) at the k-th largest tile score over the tiles
 * lying before the window.  A tile's score is the largest score of its
 * keys [P2 "Extracting block scores from exact attention": block score = maximum over the
 * block's tokens], so these are the scores of k distinct candidates and the k-th candidate score
 * is at least as large: only keys at or above the bound enter the candidate lists, and ranking
 * needs no more than that [P2 "TopK only needs ranking"].  bound_margin (log2 units, finite) is
 * subtracted from the bound to cover the two passes' different accumulation orders (1/64 is
 * ample); a row whose bound still exceeds its k-th score collects fewer than k candidates and is
 * selected again without it, so the index sets never depend on the bound or the margin (a
 * negative margin only costs that second pass).  Other shapes run the two calls one after the
 * other.  Workspace: hs_workspace_size(HS_OP_FULL_ATTN_TOPK, desc, k_global, window). */
hs_status hs_full_attn_topk(const hs_attn_desc* desc, const void* q, const void* k, const void* v,
                            int32_t k_global, int32_t window, float bound_margin, void* o,
                            float* lse, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                            void* stream);

/* Sparse layer over the full layer's K, V and index set, with the layer's own queries q
 * [P2 "Cross-layer KV cache reuse", gather equations; P2 "Same query, two memories";
 * P4 section 3.3].
 *   kind == HS_IDX_TOKEN: idx [B, q_len, Hkv, idx_cap] distinct token positions (ascending or
 *     not), the first count[b,j,u] entries valid; attention over exactly those keys.
 *   kind == HS_IDX_BLOCK: idx [B, q_len, Hkv, idx_cap] block ids, count valid; attention over
 *     the keys of those blocks (size `block`), masked causally inside a block that crosses t
 *     [P2 engineering constraint 4].
 *   swa != NULL (HySparse): adds the sliding-window branch over swa->k_local/v_local and returns
 *     sigmoid(zG) * o_glob + sigmoid(zL) * o_loc.  swa == NULL (HySparse2): returns o_glob.
 * Entries must lie in 0..t (tokens) or 0..t/block (blocks); entries outside are masked out.
 * o: [B, q_len, Hq, d] out_dtype.  lse_opt (nullable): [B, Hq, q_len] LSE of the global branch. */
hs_status hs_sparse_attn_gather(const hs_attn_desc* desc, const void* q, const void* k_full,
                                const void* v_full, hs_index_kind kind, const int32_t* idx,
                                const int32_t* count, int32_t idx_cap, int32_t block,
                                const hs_swa_branch* swa, void* o, float* lse_opt, void* ws,
                                size_t ws_bytes, void* stream);

/* ---- Selection from stored logits (decode) ------------------------------------------------
 * With few query rows per call, full attention can keep the logits it computes, so that the
 * index selection reads them back instead of recomputing them from Q and K.  The pages allow
 * either way of getting the normalized scores: computing them once the LSE is known, in a
 * second pass, or from values kept during the attention pass [P2 "Why normalize scores for
 * TopK" and "Extracting block scores from exact attention"].  The result is the same index set;
 * the traffic changes: per (b, t, u) the scores cost 4 g bytes per key written and read back,
 * against 2 d bytes of K re-read per key.  Meant for decode (q_len of a few rows): the logit
 * array holds B * q_len * Hq * kv_len floats. */

/* hs_full_attn_fwd that also stores every dot product q_t . k_i it computes (fp32, before the
 * scale tau) to logits: [B, q_len, Hq, kv_len] fp32, caller-owned, 4-byte aligned (16 for
 * full-width stores).  Entries i <= t of query row t are the attention logits times sqrt(d);
 * entries past t are unspecified (those of the last query row's range are written, larger ones
 * not).  Always runs on the split row kernel (the group kernel for groups of 32-64 heads with
 * bf16 inputs and head_dim 128 or 256; groups above 16 heads), whatever q_len is; o and lse are
 * bit-identical to what hs_full_attn_fwd returns for the same inputs on that kernel (whenever
 * hs_full_attn_fwd does not take the tiled prefill kernel: q_len * g <= 16, fp32 inputs, groups
 * above 16 with fewer than 128 query rows per KV head, or groups that do not divide the tiled
 * kernel's rows).  Workspace: hs_workspace_size(HS_OP_FULL_ATTN_LOGITS, ...). */
hs_status hs_full_attn_fwd_logits(const hs_attn_desc* desc, const void* q, const void* k,
                                  const void* v, void* o, float* lse, float* logits, void* ws,
                                  size_t ws_bytes, void* stream);

/* hs_oracle_topk with the scores taken from logits (as stored by hs_full_attn_fwd_logits for the
 * same desc) and lse instead of Q and K: same index set, same layout and padding of idx and
 * count.  desc->in_dtype is not used; desc->scale (0: 1/sqrt(head_dim)) scales the logits.
 * Any group size g <= 64.  Workspace: hs_workspace_size(HS_OP_TOPK_FROM_LOGITS, desc, k_global, window). */
hs_status hs_oracle_topk_from_logits(const hs_attn_desc* desc, const float* logits,
                                     const float* lse, int32_t k_global, int32_t window,
                                     int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                                     void* stream);

/* hs_block_score_topk with the block scores taken from logits and lse: same blocks, layout and
 * padding.  Any group size g <= 64; block a multiple of 16; 1 <= n_blocks <= 64.  Workspace:
 * hs_workspace_size(HS_OP_BLOCK_TOPK_FROM_LOGITS, desc, block, n_blocks). */
hs_status hs_block_topk_from_logits(const hs_attn_desc* desc, const float* logits,
                                    const float* lse, int32_t block, int32_t n_blocks,
                                    int32_t* blk_idx, int32_t* count, void* ws, size_t ws_bytes,
                                    void* stream);

/* hs_full_attn_fwd over a paged K / V cache, optionally keeping the logits like
 * hs_full_attn_fwd_logits (logits may be NULL).  Decode and prefill take different kernels, as
 * the pages require of a paged cache [P2 engineering constraints 2 and 3]:
 *   - logits == NULL, a prefill shape (one that hs_full_attn_fwd runs on the tiled prefill
 *     kernel) and page_size >= the kernel's key tile (64 keys; 32 at head_dim 256): the tiled
 *     prefill kernel, which reads each key tile from its page (a page holds whole tiles); o and
 *     lse are bit-identical to hs_full_attn_fwd's for the same logical cache.
 *   - otherwise the split row kernel (meant for decode), which translates every key: same o,
 *     lse (and logits) as the contiguous call on that kernel, bit for bit, except for groups of
 *     32-64 heads, whose contiguous call runs the group kernel: there the logits are identical
 *     and o, lse agree to rounding (other split boundaries).
 * Workspace: hs_workspace_size(HS_OP_FULL_ATTN_PAGED, desc, page_size, logits != NULL) (0 on
 * the prefill kernel). */
hs_status hs_full_attn_fwd_paged(const hs_attn_desc* desc, const void* q, const void* k_pool,
                                 const void* v_pool, const hs_kv_pages* pages, void* o, float* lse,
                                 float* logits, void* ws, size_t ws_bytes, void* stream);

/* hs_oracle_topk and hs_block_score_topk over a paged K cache (prefill over a paged cache):
 * the same index sets as the contiguous calls on the same logical cache, bit for bit, from the
 * streamed prefill selection, which reads every 64-key tile of K from its page.  Prefill shapes
 * only (those the contiguous calls run on that selection: many query rows per KV head), with
 * page_size >= 64 (pages hold whole tiles); other shapes or smaller pages: HS_ERR_UNSUPPORTED
 * (decode selects from the logits that hs_full_attn_fwd_paged keeps, which never read the
 * pages) [P2 engineering constraints 2 and 3: the block table is consumed by the kernel; prefill
 * and decode have their own implementations].  NULL pages: HS_ERR_INVALID_ARG.  Workspace: as
 * the contiguous call (HS_OP_ORACLE_TOPK / HS_OP_BLOCK_TOPK). */
hs_status hs_oracle_topk_paged(const hs_attn_desc* desc, const void* q, const void* k_pool,
                               const hs_kv_pages* pages, const float* lse, int32_t k_global,
                               int32_t window, int32_t* idx, int32_t* count, void* ws,
                               size_t ws_bytes, void* stream);
hs_status hs_block_score_topk_paged(const hs_attn_desc* desc, const void* q, const void* k_pool,
                                    const hs_kv_pages* pages, const float* lse, int32_t block,
                                    int32_t n_blocks, int32_t* blk_idx, int32_t* count, void* ws,
                                    size_t ws_bytes, void* stream);

/* hs_sparse_attn_gather_ex over a paged K / V cache (token and block index sets address logical
 * positions; the sliding-window branch keeps its own position-indexed or ring cache).  Same
 * outputs as the contiguous call (bit for bit; to rounding for groups of 32-64 heads, whose
 * contiguous call runs the group kernel).  Workspace: HS_OP_SPARSE_ATTN, as the contiguous
 * call (that size covers both). */
hs_status hs_sparse_attn_gather_paged(const hs_attn_desc* desc, const void* q, const void* k_pool,
                                      const void* v_pool, const hs_kv_pages* pages,
                                      hs_index_kind kind, const int32_t* idx,
                                      const int32_t* count, int32_t idx_cap, int32_t block,
                                      const hs_swa_branch* swa, const hs_sparse_opts* opts,
                                      void* o, float* lse_opt, void* ws, size_t ws_bytes,
                                      void* stream);

/* hs_sparse_attn_gather with options (opts may be NULL: then it is hs_sparse_attn_gather).
 * sink_local requires swa.  Workspace: as hs_sparse_attn_gather (HS_OP_SPARSE_ATTN). */
hs_status hs_sparse_attn_gather_ex(const hs_attn_desc* desc, const void* q, const void* k_full,
                                   const void* v_full, hs_index_kind kind, const int32_t* idx,
                                   const int32_t* count, int32_t idx_cap, int32_t block,
                                   const hs_swa_branch* swa, const hs_sparse_opts* opts, void* o,
                                   float* lse_opt, void* ws, size_t ws_bytes, void* stream);

/* hs_sparse_attn_gather without a workspace argument, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid allocation).
 * Same kernels and outputs, bit for bit, as hs_sparse_attn_gather with the same arguments; the
 * split partials live in a device-resident scratch array that the library holds for the life of
 * the process, one copy per device, 16 MiB each (a layer that needs more, i.e. more than
 * hs_workspace_size(HS_OP_SPARSE_ATTN, ...) = 16 MiB, returns HS_ERR_WORKSPACE; decode-shaped
 * layers of the pages' workloads need under 5 MiB).  Allocates nothing.  `stream` must belong to
 * the current device.  Every call on a device shares that device's scratch: calls that overlap
 * on one device (different streams, threads) race and must be serialized by the caller. */
hs_status hs_sparse_attn_gather_noalloc(const hs_attn_desc* desc, const void* q,
                                        const void* k_full, const void* v_full,
                                        hs_index_kind kind, const int32_t* idx,
                                        const int32_t* count, int32_t idx_cap, int32_t block,
                                        const hs_swa_branch* swa, void* o, float* lse_opt,
                                        void* stream);

/* Bytes of workspace the call `op` needs for `desc` (p0, p1 as documented on hs_op).  Returns 0
 * for an invalid description (hs_last_error() says why). */
size_t hs_workspace_size(hs_op op, const hs_attn_desc* desc, int32_t p0, int32_t p1);

const char* hs_status_string(hs_status s);

/* Thread-local description of the last non-OK return on this thread ("" if none). */
const char* hs_last_error(void);

/* Library version string. */
const char* hs_version(void);

#ifdef __cplusplus
}
#endif
#endif
