/*
 * hs_oracle.h -- plain CPU reference for the HySparse / HySparse2 attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls this code;
 * only the test-suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * source, header, table or helper with the GPU library.
 *
 * Everything is computed in IEEE double from float inputs (the exact values the GPU sees, bf16
 * values widened exactly to float).  No blocking, fusion or reordering beyond the definitions:
 * every row is evaluated from its definition with a plain loop over all keys.
 *
 * Sources (web pages; sections cited in each function's comment):
 *   [P1] "HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing" -- reading notes,
 *        qqtang-code.github.io (Chinese).
 *   [P2] "HySparse hybrid sparse attention (part 1): full attention as the oracle" --
 *        pinghaoyang.com.cn (Chinese); the most detailed statement of the equations.
 *   [P4] "HySparse: A Hybrid Sparse Attention Architecture with Oracle Token Selection and KV
 *        Cache Sharing" -- papercache.org summary of arXiv:2602.03560.
 *   [P5] "HySparse2: Hybrid Sparse Attention with Two-Level KV Sharing" -- picx.dev summary.
 *
 * Layouts (row-major, head_dim fastest):
 *   Q, O, Q' : [B, Tq, Hq, d]     K, V, K', V' : [B, Tk, Hkv, d]     LSE : [B, Hq, Tq]
 *   idx      : [B, Tq, Hkv, cap]  count        : [B, Tq, Hkv]       gate : [B, Tq, Hq, 2]
 * Query row j sits at absolute position t = q_offset + j; it may attend keys 0..t.
 * Query head h reads KV head u = h / g with g = Hq / Hkv (contiguous grouping).
 *
 * Row subsets: every per-row function takes (rows, n_rows).  rows == NULL means every query row
 * 0..Tq-1; otherwise only the listed query rows are evaluated (for all batches and heads) and all
 * other output entries are left untouched.  This is how large workloads are sampled.
 *
 * Return value of every function: 0 on success, a negative code on invalid arguments
 * (ORC_EINVAL) or when an index set holds an entry outside [0, t] (ORC_EINDEX).
 */
#ifndef HS_ORACLE_H
#define HS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_EINDEX (-2)

typedef struct {
  int32_t batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim;
  int64_t q_offset; /* absolute position of query row 0; q_offset + q_len <= kv_len */
  double scale;     /* logit scale tau; 0 means 1/sqrt(head_dim) */
} orc_shape;

/* Worker threads used by the parallel row loops (0 = OpenMP default). Returns the count in use. */
int orc_set_threads(int n);
int orc_threads(void);

/* Logits a_{t,i} = tau q_t . k_i (tau = scale, or 1/sqrt(d) when scale is 0), i = 0..t, of one
 * (b, j, h).  a must hold t+1 doubles. */
int orc_logit_row(const orc_shape* s, const float* q, const float* k, int b, int j, int h,
                  double* a);

/* Per-head normalized probabilities p_{t,i} = exp(a_{t,i} - LSE_t), i = 0..t, for one
 * (b, j, h).  lse may be NULL (then LSE is recomputed from the row).  p must hold t+1 doubles. */
int orc_prob_row(const orc_shape* s, const float* q, const float* k, const double* lse, int b,
                 int j, int h, double* p);

/* Full causal GQA attention: O (double) and LSE = ln sum_{i<=t} exp(a_{t,i}). */
int orc_full_attention(const orc_shape* s, const float* q, const float* k, const float* v,
                       double* o, double* lse, const int32_t* rows, int n_rows);

/* Token score of every key i <= t for one (b, j, u): s_i = max over the group's heads of p. */
int orc_token_score_row(const orc_shape* s, const float* q, const float* k, const double* lse,
                        int b, int j, int u, double* score);

/* Token index set: forced window {max(0,t-w+1)..t} plus the k_global best-scoring keys among
 * 0..t-w, ranked by (score desc, position asc).  Output ascending, -1 padded to cap. */
int orc_token_topk(const orc_shape* s, const float* q, const float* k, const double* lse,
                   int k_global, int window, int cap, int32_t* idx, int32_t* count,
                   const int32_t* rows, int n_rows);

/* Attention of Q' over K, V restricted to the index set of (b, j, u): dense masked softmax over
 * all keys 0..t with non-members at -inf.  lse may be NULL. */
int orc_masked_attention(const orc_shape* s, const float* q, const float* k, const float* v,
                         const int32_t* idx, const int32_t* count, int cap, double* o,
                         double* lse, const int32_t* rows, int n_rows);

/* orc_masked_attention with a per-head sink logit (sink [Hq], NULL: none) in the softmax
 * denominator, LSE = ln(e^{s_h} + sum_{i in I} e^{a_i}), and a sigmoid output gate
 * (out_gate [B, Tq, Hq] logits, NULL: none) applied to the result. */
int orc_masked_attention_ex(const orc_shape* s, const float* q, const float* k, const float* v,
                            const int32_t* idx, const int32_t* count, int cap, const float* sink,
                            const float* out_gate, double* o, double* lse, const int32_t* rows,
                            int n_rows);

/* orc_masked_attention_ex with a per-channel output gate out_gate_ch [B, Tq, Hq, d] (logits;
 * channel c of the output is scaled by sigmoid(out_gate_ch[.., c])). */
int orc_masked_attention_ch(const orc_shape* s, const float* q, const float* k, const float* v,
                            const int32_t* idx, const int32_t* count, int cap, const float* sink,
                            const float* out_gate_ch, double* o, double* lse,
                            const int32_t* rows, int n_rows);

/* Block score of every causal block r = 0..floor(t/B) for one (b, j, u):
 * max over heads of max over i in [rB, min(rB+B-1, t)] of p^h_{t,i}. */
int orc_block_score_row(const orc_shape* s, const float* q, const float* k, const double* lse,
                        int b, int j, int u, int block, double* score);

/* Top n_blocks causal blocks by (score desc, block id asc); ascending, -1 padded to n_blocks. */
int orc_block_topk(const orc_shape* s, const float* q, const float* k, const double* lse,
                   int block, int n_blocks, int32_t* blk_idx, int32_t* count,
                   const int32_t* rows, int n_rows);

/* HySparse sparse layer: block-sparse branch over K, V (selected blocks, causal inside the block)
 * plus a sliding-window branch over the layer's own K', V' (positions max(0,t-w+1)..t), combined
 * with per-head sigmoid gates: o = sigmoid(zG) o_glob + sigmoid(zL) o_loc.  o_glob / o_loc may be
 * NULL; when given they receive the two branch outputs. */
int orc_gated_block_swa(const orc_shape* s, const float* q, const float* k, const float* v,
                        const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                        const float* k_loc, const float* v_loc, int window, const float* gate,
                        double* o, double* o_glob, double* o_loc, const int32_t* rows,
                        int n_rows);

/* orc_gated_block_swa with a per-head sink in the global (sink) and local (sink_loc) branch and
 * a sigmoid output gate on the gated sum; any of the three may be NULL. */
int orc_gated_block_swa_ex(const orc_shape* s, const float* q, const float* k, const float* v,
                           const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                           const float* k_loc, const float* v_loc, int window, const float* gate,
                           const float* sink, const float* sink_loc, const float* out_gate,
                           double* o, double* o_glob, double* o_loc, const int32_t* rows,
                           int n_rows);

/* orc_gated_block_swa_ex with per-channel gates: gate_ch [B, Tq, Hq, 2, d] holds the d logits of
 * zG then the d of zL for each (query, head); out_gate_ch [B, Tq, Hq, d] (or NULL) gates the sum
 * per channel.  o_c = sigmoid(out_c) (sigmoid(zG_c) o_glob,c + sigmoid(zL_c) o_loc,c). */
int orc_gated_block_swa_ch(const orc_shape* s, const float* q, const float* k, const float* v,
                           const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                           const float* k_loc, const float* v_loc, int window,
                           const float* gate_ch, const float* sink, const float* sink_loc,
                           const float* out_gate_ch, double* o, double* o_glob, double* o_loc,
                           const int32_t* rows, int n_rows);

#ifdef __cplusplus
}
#endif
#endif
