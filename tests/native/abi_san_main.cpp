// Host-sanitizer driver of the C ABI's host code (test infrastructure): the library's sources are
// compiled for the host only, with AddressSanitizer and UndefinedBehaviorSanitizer, and this
// program runs the argument checks, the workspace-size and launch-geometry arithmetic over a
// grid of shapes (every group size up to 64, head sizes 64-256, short and long contexts) and,
// only when no GPU is visible, the valid calls up to their (failing) launch.  Any undefined
// arithmetic (a division by zero, an overflow, an out-of-bounds access) aborts the run.
// Prints "OK" on success.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "hysparse.h"

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                      \
    }                                                                \
  } while (0)

static hs_attn_desc make(int B, int Tq, int Tk, int Hq, int Hkv, int d, hs_dtype in = HS_BF16) {
  hs_attn_desc x;
  x.batch = B;
  x.q_len = Tq;
  x.kv_len = Tk;
  x.n_q_heads = Hq;
  x.n_kv_heads = Hkv;
  x.head_dim = d;
  x.q_offset = -1;
  x.scale = 0.f;
  x.in_dtype = in;
  x.out_dtype = HS_F32;
  return x;
}

int main() {
  void* const F = (void*)0x1000;  // never dereferenced on the host
  int32_t* const FI = (int32_t*)0x1000;
  float* const FF = (float*)0x1000;
  const int groups[] = {1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 40, 48, 56, 64};
  const int dims[] = {64, 128, 256};
  const int qlens[] = {1, 3, 100, 4096};
  const int klens[] = {100, 5000, 135168, 1 << 20};
  size_t total = 0;
  for (int g : groups)
    for (int d : dims)
      for (int Tq : qlens)
        for (int Tk : klens) {
          if (Tq > Tk) continue;
          const hs_attn_desc x = make(4, Tq, Tk, g * 2, 2, d);
          for (int op = 0; op <= 8; op++) {
            int p0 = 0, p1 = 0;
            if (op == HS_OP_ORACLE_TOPK || op == HS_OP_TOPK_FROM_LOGITS) p0 = 1024, p1 = 128;
            if (op == HS_OP_BLOCK_TOPK || op == HS_OP_BLOCK_TOPK_FROM_LOGITS ||
                op == HS_OP_FULL_ATTN_BLOCK_TOPK)
              p0 = 64, p1 = 16;
            if (op == HS_OP_SPARSE_ATTN) p0 = 1152, p1 = 128;
            if (op == HS_OP_FULL_ATTN_PAGED) p0 = 64;
            total += hs_workspace_size((hs_op)op, &x, p0, p1);
          }
        }
  std::printf("workspace sizes summed: %zu\n", total);

  // invalid descriptions and arguments: rejected before anything is enqueued
  hs_attn_desc x = make(1, 1, 1024, 8, 2, 128);
  x.head_dim = 96;
  CHECK(hs_full_attn_fwd(&x, F, F, F, F, FF, F, 1 << 30, nullptr) == HS_ERR_UNSUPPORTED);
  x = make(1, 1, 1024, 8, 2, 128);
  x.scale = -1.f;
  CHECK(hs_full_attn_fwd(&x, F, F, F, F, FF, F, 1 << 30, nullptr) == HS_ERR_INVALID_ARG);
  x = make(1, 1, 1024, 6, 4, 128);
  CHECK(hs_full_attn_fwd(&x, F, F, F, F, FF, F, 1 << 30, nullptr) == HS_ERR_INVALID_ARG);
  x = make(1, 4, 1024, 8, 2, 128);
  x.q_offset = 1021;
  CHECK(hs_oracle_topk(&x, F, F, FF, 1024, 128, FI, FI, F, 1 << 30, nullptr) ==
        HS_ERR_INVALID_ARG);
  x = make(1, 1, 1024, 8, 2, 128);
  CHECK(hs_oracle_topk(&x, F, F, FF, -1, 128, FI, FI, F, 1 << 30, nullptr) == HS_ERR_INVALID_ARG);
  CHECK(hs_block_score_topk(&x, F, F, FF, 24, 16, FI, FI, F, 1 << 30, nullptr) ==
        HS_ERR_UNSUPPORTED);
  hs_swa_branch swa = {F, F, FF, 128};
  hs_sparse_opts opts = {nullptr, nullptr, nullptr, 130};
  x = make(1, 4, 1024, 8, 2, 128);
  CHECK(hs_sparse_attn_gather_ex(&x, F, F, F, HS_IDX_BLOCK, FI, FI, 16, 64, &swa, &opts, F,
                                 nullptr, F, 1 << 30, nullptr) == HS_ERR_INVALID_ARG);
  hs_sparse_opts opts_ch = {nullptr, nullptr, nullptr, 0, 3};  // gates_per_channel is 0 or 1
  CHECK(hs_sparse_attn_gather_ex(&x, F, F, F, HS_IDX_BLOCK, FI, FI, 16, 64, &swa, &opts_ch, F,
                                 nullptr, F, 1 << 30, nullptr) == HS_ERR_INVALID_ARG);
  hs_kv_pages pages = {FI, 48, 32, 100};  // not a power of two
  CHECK(hs_full_attn_fwd_paged(&x, F, F, F, &pages, F, FF, nullptr, F, 1 << 30, nullptr) ==
        HS_ERR_INVALID_ARG);
  // paged selection: prefill shapes on pages of at least 64 positions only
  hs_kv_pages small = {FI, 32, 128, 256};
  x = make(1, 512, 4096, 16, 4, 128);
  CHECK(hs_oracle_topk_paged(&x, F, F, &small, FF, 256, 64, FI, FI, F, 1 << 30, nullptr) ==
        HS_ERR_UNSUPPORTED);
  CHECK(hs_block_score_topk_paged(&x, F, F, nullptr, FF, 64, 16, FI, FI, F, 1 << 30, nullptr) ==
        HS_ERR_INVALID_ARG);
  hs_kv_pages p64 = {FI, 64, 64, 64};
  x = make(1, 1, 4096, 16, 4, 128);
  CHECK(hs_oracle_topk_paged(&x, F, F, &p64, FF, 256, 64, FI, FI, F, 1 << 30, nullptr) ==
        HS_ERR_UNSUPPORTED);

  // valid calls reach their launch, which fails without a GPU; never run with one visible
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess || n_dev == 0) {
    for (int g : groups)
      for (int Tq : {1, 200}) {
        hs_attn_desc y = make(2, Tq, 3000, 2 * g, 2, 128);
        const size_t big = (size_t)1 << 40;
        hs_full_attn_fwd(&y, F, F, F, F, FF, F, big, nullptr);
        hs_oracle_topk(&y, F, F, FF, 256, 64, FI, FI, F, big, nullptr);
        hs_block_score_topk(&y, F, F, FF, 64, 16, FI, FI, F, big, nullptr);
        hs_sparse_attn_gather(&y, F, F, F, HS_IDX_TOKEN, FI, FI, 320, 64, nullptr, F, FF, F, big,
                              nullptr);
        hs_sparse_attn_gather(&y, F, F, F, HS_IDX_BLOCK, FI, FI, 16, 64, &swa, F, FF, F, big,
                              nullptr);
        hs_oracle_topk_from_logits(&y, FF, FF, 256, 64, FI, FI, F, big, nullptr);
        hs_block_topk_from_logits(&y, FF, FF, 64, 16, FI, FI, F, big, nullptr);
        hs_full_attn_fwd_logits(&y, F, F, F, F, FF, FF, F, big, nullptr);
        hs_sparse_attn_gather_noalloc(&y, F, F, F, HS_IDX_TOKEN, FI, FI, 320, 64, nullptr, F, FF,
                                      nullptr);
        hs_kv_pages pg = {FI, 64, 47, 200};
        hs_full_attn_fwd_paged(&y, F, F, F, &pg, F, FF, nullptr, F, big, nullptr);
        hs_oracle_topk_paged(&y, F, F, &pg, FF, 256, 64, FI, FI, F, big, nullptr);
        hs_block_score_topk_paged(&y, F, F, &pg, FF, 64, 16, FI, FI, F, big, nullptr);
      }
    std::printf("valid calls exercised without a GPU\n");
  }
  std::printf("OK\n");
  return 0;
}
