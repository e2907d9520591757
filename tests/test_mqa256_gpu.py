"""GPU parity for HySparse2's own head shape (MQA: 64 query heads on one KV head, d 256) and for
other GQA groups larger than 16, which the kernels run as chunks of 16 heads: full attention,
selection from stored logits, token-sparse and gated block-sparse layers, paged cache, against
the CPU oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import LSE_TOL, TOL_BF16, check_block_sets, check_token_sets, max_abs

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


SHAPES = [
    ("mqa64_d256_decode", Workload("m", 2, 1, 5000, 64, 1, 256, "bf16", k_global=1024,
                                   window=128, block=64, n_blocks=16, needles=4, seed=701)),
    ("mqa64_d256_three_queries", Workload("m3", 1, 3, 2100, 64, 1, 256, "bf16", k_global=300,
                                          window=64, block=64, n_blocks=8, seed=702)),
    ("g32_d128_decode", Workload("g32", 2, 1, 4000, 64, 2, 128, "bf16", k_global=512, window=64,
                                 block=64, n_blocks=16, seed=703)),
    ("g48_d64_decode", Workload("g48", 1, 1, 3000, 48, 1, 64, "bf16", k_global=256, window=32,
                                block=32, n_blocks=12, seed=704)),
    # three 16-head chunks per workgroup, two queries, a ragged key count (scalar logit stores)
    ("g48_d128_two_queries_ragged", Workload("g48b", 1, 2, 3001, 48, 1, 128, "bf16", k_global=256,
                                             window=32, block=64, n_blocks=8, seed=705)),
    ("g32_d256_decode_odd", Workload("g32c", 1, 1, 2999, 32, 1, 256, "bf16", k_global=512,
                                     window=64, block=64, n_blocks=16, seed=706)),
]


@pytest.mark.parametrize("name,wl", SHAPES, ids=[s[0] for s in SHAPES])
def test_full_attention_and_logits_selection(name, wl):
    say(f"[large group] {name} {wl}")
    x = make_inputs(wl, device="cuda", n_sparse=1)
    q, k, v = x["q"], x["k"], x["v"]
    o, lse, lg = hs().full_attn_fwd_logits(q, k, v, out_dtype=torch.float32)
    o2, lse2 = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
    idx, cnt = hs().oracle_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.k_global,
                                            wl.window)
    bi, bc = hs().block_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.block,
                                         wl.n_blocks)
    torch.cuda.synchronize()
    if wl.q_len * wl.n_q_heads // wl.n_kv_heads < 128:
        assert torch.equal(o, o2) and torch.equal(lse, lse2)  # the same split kernel
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.full_attention(qn, kn, vn)
    eo, el = max_abs(o.cpu().numpy(), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    say(f"  full attention max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
    assert eo <= TOL_BF16 and el <= LSE_TOL
    # without logits, many query rows run the tiled prefill kernel
    eo2, el2 = max_abs(o2.cpu().numpy(), o_ref), max_abs(lse2.cpu().numpy(), lse_ref)
    assert eo2 <= TOL_BF16 and el2 <= LSE_TOL
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    ex = check_token_sets(idx.cpu().numpy(), cnt.cpu().numpy(), oi, oc, qn, kn, lse_ref,
                          wl.k_global, wl.window, wl.q_offset)
    say(f"  token sets: near-tie differences excused {ex}")
    if wl.needles:
        for b in range(wl.batch):
            sel = set(idx[b, -1, 0, :cnt[b, -1, 0]].cpu().tolist())
            assert set(x["needle_pos"][b, 0].tolist()) <= sel
    obi, obc = oracle.block_topk(qn, kn, lse_ref, wl.block, wl.n_blocks)
    ex = check_block_sets(bi.cpu().numpy(), bc.cpu().numpy(), obi, obc, qn, kn, lse_ref,
                          wl.block, wl.q_offset)
    say(f"  block sets: near-tie differences excused {ex}")
    # the token-sparse layer over the oracle's sets, with a sink
    g = torch.Generator().manual_seed(wl.seed)
    sink = torch.randn(wl.n_q_heads, generator=g)
    qs = x["q_sparse"][0]
    os_, ls_ = hs().sparse_attn_gather(qs, k, v, torch.from_numpy(oi).cuda(),
                                       torch.from_numpy(oc).cuda(), kind="token",
                                       out_dtype=torch.float32, want_lse=True, sink=sink.cuda())
    torch.cuda.synchronize()
    r_o, r_l = oracle.masked_attention(to_numpy_f32(qs), kn, vn, oi, oc, sink=sink.numpy())
    eo, el = max_abs(os_.cpu().numpy(), r_o), max_abs(ls_.cpu().numpy(), r_l)
    say(f"  token-sparse max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
    assert eo <= TOL_BF16 and el <= LSE_TOL


@pytest.mark.parametrize("name,wl", SHAPES[:3], ids=[s[0] for s in SHAPES[:3]])
def test_gated_layer_large_groups(name, wl):
    x = make_inputs(wl, device="cuda", block_variant=True)
    a = {n: to_numpy_f32(x[n]) for n in ("q", "k", "v", "k_loc", "v_loc", "gate")}
    qs = x["q_sparse"][0]
    bi, bc = oracle.block_topk(a["q"], a["k"], None, wl.block, wl.n_blocks)
    g = torch.Generator().manual_seed(wl.seed + 1)
    s1, s2 = torch.randn(wl.n_q_heads, generator=g), torch.randn(wl.n_q_heads, generator=g)
    o_ref, _, _ = oracle.gated_block_swa(to_numpy_f32(qs), a["k"], a["v"], bi, bc, wl.block,
                                         a["k_loc"], a["v_loc"], wl.window, a["gate"],
                                         sink=s1.numpy(), sink_loc=s2.numpy())
    o, _ = hs().sparse_attn_gather(qs, x["k"], x["v"], torch.from_numpy(bi).cuda(),
                                   torch.from_numpy(bc).cuda(), kind="block", block=wl.block,
                                   swa=(x["k_loc"], x["v_loc"], x["gate"], wl.window),
                                   out_dtype=torch.float32, sink=s1.cuda(), sink_local=s2.cuda())
    torch.cuda.synchronize()
    eo = max_abs(o.cpu().numpy(), o_ref)
    say(f"[gated large group] {name} max|dO| = {eo:.3e}")
    assert eo <= TOL_BF16


def test_prefill_kernel_with_64_heads_per_kv_head():
    wl = Workload("pf64", 1, 40, 1500, 64, 1, 128, "bf16", seed=711)
    x = make_inputs(wl, device="cuda")
    o, lse = hs().full_attn_fwd(x["q"], x["k"], x["v"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full_attention(*(to_numpy_f32(x[n]) for n in ("q", "k", "v")))
    eo, el = max_abs(o.cpu().numpy(), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    say(f"[prefill g=64] max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
    assert eo <= TOL_BF16 and el <= LSE_TOL


def test_paged_mqa256_equals_contiguous():
    from test_paged_gpu import paged
    wl = Workload("pm", 2, 1, 3000, 64, 1, 256, "bf16", seed=721)
    x = make_inputs(wl, device="cuda", n_sparse=1)
    kp, table = paged(x["k"], 32, 721)
    vp, _ = paged(x["v"], 32, 721)
    o, lse, lg = hs().full_attn_fwd_logits(x["q"], x["k"], x["v"], out_dtype=torch.float32)
    o2, lse2, lg2 = hs().full_attn_fwd_paged(x["q"], kp, vp, table, wl.kv_len, logits=True,
                                             out_dtype=torch.float32)
    idx, cnt = hs().oracle_topk_from_logits(lg, lse, 1, 256, wl.k_global, wl.window)
    s1, _ = hs().sparse_attn_gather(x["q_sparse"][0], x["k"], x["v"], idx, cnt,
                                    out_dtype=torch.float32)
    s2, _ = hs().sparse_attn_gather(x["q_sparse"][0], kp, vp, idx, cnt, pages=(table, wl.kv_len),
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the logits are the same dot products; over a paged cache full attention and the sparse
    # layer run the row kernel, the contiguous calls the group kernel: other split boundaries,
    # so P is rounded to bf16 against other running maxima (the LSE sums fp32 exponentials)
    assert torch.equal(lg, lg2)
    assert (o - o2).abs().max().item() <= TOL_BF16
    assert (lse - lse2).abs().max().item() <= LSE_TOL
    assert (s1 - s2).abs().max().item() <= TOL_BF16


def test_unsupported_combinations_are_rejected():
    """Head size 256 takes bf16 inputs only: fp32 calls are refused before any launch (the
    selection calls included, which accept every group size and head size 256 in bf16)."""
    wl = Workload("rj", 1, 1, 500, 64, 1, 256, "f32", seed=731)
    x = make_inputs(wl, device="cuda")
    lse = torch.zeros((1, 64, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(hs().HsError):
        hs().full_attn_fwd(x["q"], x["k"], x["v"])
    with pytest.raises(hs().HsError):
        hs().oracle_topk(x["q"], x["k"], lse, 64, 16)
    with pytest.raises(hs().HsError):
        hs().block_score_topk(x["q"], x["k"], lse, 64, 4)


@pytest.mark.parametrize("with_sink", [False, True], ids=["no_sink", "sink"])
def test_group_kernel_empty_and_partial_index_sets(with_sink):
    """Token sets of 64 heads on one KV head (the group kernel): a set with count 0 attends over
    nothing (output 0; LSE -inf, or the sink when there is one), a set with a few entries and -1
    padding inside its count as usual."""
    wl = Workload("ge", 2, 2, 1500, 64, 1, 256, "bf16", k_global=200, window=32, seed=741)
    x = make_inputs(wl, device="cuda", n_sparse=1)
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    oi, oc = oracle.token_topk(qn, kn, None, wl.k_global, wl.window)
    oc = oc.copy()
    oc[1, 0, 0] = 0                       # empty set
    # padding inside the count: the GPU skips those entries; the oracle, whose sets hold valid
    # positions only, gets the same set without them
    gi = oi.copy()
    gi[0, 1, 0, 3:7] = -1
    n = oc[0, 1, 0]
    oi = oi.copy()
    oi[0, 1, 0, :n - 4] = np.concatenate([oi[0, 1, 0, :3], oi[0, 1, 0, 7:n]])
    oi[0, 1, 0, n - 4:] = -1
    gc = oc.copy()
    oc[0, 1, 0] = n - 4
    sink = torch.randn(wl.n_q_heads, generator=torch.Generator().manual_seed(742)) if with_sink else None
    qs = x["q_sparse"][0]
    o, lse = hs().sparse_attn_gather(qs, x["k"], x["v"], torch.from_numpy(gi).cuda(),
                                     torch.from_numpy(gc).cuda(), kind="token",
                                     out_dtype=torch.float32, want_lse=True,
                                     sink=None if sink is None else sink.cuda())
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    o_ref, lse_ref = oracle.masked_attention(to_numpy_f32(qs), kn, vn, oi, oc,
                                             sink=None if sink is None else sink.numpy())
    assert (o[1, 0] == 0).all()
    if sink is None:
        assert np.isneginf(lse[1, :, 0]).all()
    else:
        assert np.allclose(lse[1, :, 0], sink.numpy(), rtol=0, atol=1e-6)
    keep = np.ones(o.shape[:2], dtype=bool)
    keep[1, 0] = False
    assert max_abs(o[keep], o_ref[keep]) <= TOL_BF16
    lk = np.isfinite(lse_ref)
    assert max_abs(lse[lk], lse_ref[lk]) <= LSE_TOL
