/* Host-sanitizer driver of the CPU oracle (test infrastructure): runs every oracle entry point on
 * small seeded inputs and on invalid arguments, in a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer, so that an out-of-bounds access or undefined arithmetic in the
 * oracle aborts the run.  Prints "OK" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "hs_oracle.h"

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double unif(void) { /* splitmix64 */
  uint64_t z = (rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return ((z >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
static float* randn(size_t n) {
  float* x = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; i++) x[i] = (float)(sqrt(-2.0 * log(unif())) * cos(6.283185307179586 * unif()));
  return x;
}
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  orc_set_threads(2);
  const int B = 2, Tq = 5, Tk = 70, Hq = 6, Hkv = 2, d = 16, kg = 7, w = 3, cap = kg + w;
  const int blk = 8, nb = 3;
  orc_shape s = {B, Tq, Tk, Hq, Hkv, d, Tk - Tq, 0.0};
  float *q = randn((size_t)B * Tq * Hq * d), *k = randn((size_t)B * Tk * Hkv * d),
        *v = randn((size_t)B * Tk * Hkv * d), *kl = randn((size_t)B * Tk * Hkv * d),
        *vl = randn((size_t)B * Tk * Hkv * d), *gate = randn((size_t)B * Tq * Hq * 2),
        *sink = randn(Hq), *sinkl = randn(Hq), *og = randn((size_t)B * Tq * Hq);
  double* o = malloc(sizeof(double) * B * Tq * Hq * d);
  double* o2 = malloc(sizeof(double) * B * Tq * Hq * d);
  double* o3 = malloc(sizeof(double) * B * Tq * Hq * d);
  double* lse = malloc(sizeof(double) * B * Hq * Tq);
  double* lse2 = malloc(sizeof(double) * B * Hq * Tq);
  int32_t* idx = malloc(sizeof(int32_t) * B * Tq * Hkv * cap);
  int32_t* cnt = malloc(sizeof(int32_t) * B * Tq * Hkv);
  int32_t* bidx = malloc(sizeof(int32_t) * B * Tq * Hkv * nb);
  int32_t* bcnt = malloc(sizeof(int32_t) * B * Tq * Hkv);
  double row[Tk];
  const int32_t rows[2] = {0, Tq - 1};

  CHECK(orc_full_attention(&s, q, k, v, o, lse, NULL, 0) == ORC_OK);
  CHECK(orc_full_attention(&s, q, k, v, o, lse, rows, 2) == ORC_OK);
  CHECK(orc_logit_row(&s, q, k, 1, Tq - 1, Hq - 1, row) == ORC_OK);
  CHECK(orc_prob_row(&s, q, k, lse, 1, 2, 3, row) == ORC_OK);
  CHECK(orc_prob_row(&s, q, k, NULL, 0, 0, 0, row) == ORC_OK);
  CHECK(orc_token_score_row(&s, q, k, lse, 1, 1, 1, row) == ORC_OK);
  CHECK(orc_token_topk(&s, q, k, lse, kg, w, cap, idx, cnt, NULL, 0) == ORC_OK);
  CHECK(orc_masked_attention(&s, q, k, v, idx, cnt, cap, o2, lse2, NULL, 0) == ORC_OK);
  CHECK(orc_masked_attention_ex(&s, q, k, v, idx, cnt, cap, sink, og, o2, lse2, rows, 2) == ORC_OK);
  CHECK(orc_block_score_row(&s, q, k, lse, 0, 4, 1, blk, row) == ORC_OK);
  CHECK(orc_block_topk(&s, q, k, lse, blk, nb, bidx, bcnt, NULL, 0) == ORC_OK);
  CHECK(orc_gated_block_swa(&s, q, k, v, bidx, bcnt, nb, blk, kl, vl, w, gate, o, o2, o3, NULL,
                            0) == ORC_OK);
  CHECK(orc_gated_block_swa_ex(&s, q, k, v, bidx, bcnt, nb, blk, kl, vl, w, gate, sink, sinkl, og,
                               o, NULL, NULL, rows, 2) == ORC_OK);
  /* per-channel gates: [B, Tq, Hq, 2, d] branch logits and a [B, Tq, Hq, d] output gate */
  {
    float *gch = randn((size_t)B * Tq * Hq * 2 * d), *ogch = randn((size_t)B * Tq * Hq * d);
    CHECK(orc_masked_attention_ch(&s, q, k, v, idx, cnt, cap, sink, ogch, o2, lse2, NULL, 0) ==
          ORC_OK);
    CHECK(orc_gated_block_swa_ch(&s, q, k, v, bidx, bcnt, nb, blk, kl, vl, w, gch, sink, sinkl,
                                 ogch, o, o2, o3, NULL, 0) == ORC_OK);
    CHECK(orc_gated_block_swa_ch(&s, q, k, v, bidx, bcnt, nb, blk, kl, vl, w, gch, NULL, NULL,
                                 NULL, o, NULL, NULL, rows, 2) == ORC_OK);
    CHECK(orc_masked_attention_ch(&s, q, k, v, idx, cnt, cap, sink, NULL, o2, lse2, NULL, 0) ==
          ORC_EINVAL);
    free(gch); free(ogch);
  }
  /* a prefill from position 0 and a non-default scale (buffers of its own size) */
  {
    orc_shape s0 = {1, 40, 40, 4, 1, 8, 0, 0.3};
    float *q0 = randn(40 * 4 * 8), *k0 = randn(40 * 8), *v0 = randn(40 * 8);
    double *oo = malloc(sizeof(double) * 40 * 4 * 8), *ll = malloc(sizeof(double) * 4 * 40);
    int32_t *ii = malloc(sizeof(int32_t) * 40 * 7), *cc = malloc(sizeof(int32_t) * 40);
    int32_t *bi = malloc(sizeof(int32_t) * 40 * 3), *bc = malloc(sizeof(int32_t) * 40);
    CHECK(orc_full_attention(&s0, q0, k0, v0, oo, ll, NULL, 0) == ORC_OK);
    CHECK(orc_token_topk(&s0, q0, k0, ll, 5, 2, 7, ii, cc, NULL, 0) == ORC_OK);
    CHECK(orc_masked_attention(&s0, q0, k0, v0, ii, cc, 7, oo, ll, NULL, 0) == ORC_OK);
    CHECK(orc_block_topk(&s0, q0, k0, ll, 4, 3, bi, bc, NULL, 0) == ORC_OK);
    free(q0); free(k0); free(v0); free(oo); free(ll); free(ii); free(cc); free(bi); free(bc);
  }

  /* invalid arguments are refused, not read past */
  orc_shape bad = s;
  bad.n_q_heads = 5;
  CHECK(orc_full_attention(&bad, q, k, v, o, lse, NULL, 0) == ORC_EINVAL);
  bad = s;
  bad.q_offset = Tk;
  CHECK(orc_full_attention(&bad, q, k, v, o, lse, NULL, 0) == ORC_EINVAL);
  bad = s;
  bad.scale = -1.0;
  CHECK(orc_full_attention(&bad, q, k, v, o, lse, NULL, 0) == ORC_EINVAL);
  const int32_t badrows[1] = {Tq};
  CHECK(orc_full_attention(&s, q, k, v, o, lse, badrows, 1) == ORC_EINVAL);
  CHECK(orc_full_attention(NULL, q, k, v, o, lse, NULL, 0) == ORC_EINVAL);
  idx[0] = Tk + 5; /* an entry past t */
  cnt[0] = 1;
  CHECK(orc_masked_attention(&s, q, k, v, idx, cnt, cap, o2, lse2, NULL, 0) == ORC_EINDEX);
  free(q); free(k); free(v); free(kl); free(vl); free(gate); free(sink); free(sinkl); free(og);
  free(o); free(o2); free(o3); free(lse); free(lse2); free(idx); free(cnt); free(bidx); free(bcnt);
  printf("OK\n");
  return 0;
}
