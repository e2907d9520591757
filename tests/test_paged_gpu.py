"""GPU parity of the paged K / V cache (hs_full_attn_fwd_paged, hs_sparse_attn_gather_paged) and
of the ring-buffered sliding-window cache: the same logical cache laid out in shuffled pages
(or a ring) must give bit-identical outputs to the contiguous calls, and the paged sparse layers
(token layer with sinks, gated layer with both sinks, ring window caches) are also compared with
the oracle on the logical cache; one paged decode pipeline is checked against the oracle end to
end.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import LSE_TOL, TOL_BF16, check_token_sets, max_abs, paged

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


FA_CASES = [
    ("decode_g4_p64", Workload("d4", 2, 1, 5000, 32, 8, 128, "bf16", seed=601), 64),
    ("decode_g16_p16_ragged", Workload("d16", 2, 1, 3001, 64, 4, 128, "bf16", seed=602), 16),
    ("short_block_d64_p256", Workload("sb", 2, 3, 777, 8, 2, 64, "bf16", seed=603), 256),
    ("tiny_f32_p32", Workload("tf", 1, 64, 300, 4, 1, 64, "f32", seed=604), 32),
    ("decode_p1", Workload("p1", 1, 1, 700, 16, 4, 128, "bf16", seed=605), 1),
    ("decode_g4_d256_p32", Workload("d256", 2, 1, 2000, 8, 2, 256, "bf16", seed=607), 32),
    # a long split: many pages staged per workgroup
    ("decode_g4_70k_p16", Workload("dl", 1, 1, 70000, 32, 8, 128, "bf16", seed=606), 16),
]


@pytest.mark.parametrize("name,wl,P", FA_CASES, ids=[c[0] for c in FA_CASES])
def test_paged_full_attention_equals_contiguous(name, wl, P):
    say(f"[paged full attention] {name} {wl} page {P}")
    x = make_inputs(wl, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    kp, table = paged(k, P, wl.seed)
    vp, _ = paged(v, P, wl.seed)
    o, lse, lg = hs().full_attn_fwd_logits(q, k, v, out_dtype=torch.float32)
    o2, lse2, lg2 = hs().full_attn_fwd_paged(q, kp, vp, table, wl.kv_len, logits=True,
                                             out_dtype=torch.float32)
    o3, lse3 = hs().full_attn_fwd_paged(q, kp, vp, table, wl.kv_len, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(o, o3)
    assert torch.equal(lse, lse3)
    t = wl.q_offset + torch.arange(wl.q_len, device="cuda")
    causal = (torch.arange(wl.kv_len, device="cuda")[None, :] <= t[:, None])[None, :, None, :]
    assert torch.equal(lg.masked_fill(~causal, 0), lg2.masked_fill(~causal, 0))


SPARSE_CASES = [
    ("decode_g4_split_p64", Workload("s4", 2, 1, 6000, 32, 8, 128, "bf16", seed=611), 64),
    ("decode_g4_wide_p16", Workload("sw", 16, 1, 3000, 32, 8, 128, "bf16", seed=612), 16),
    ("prefill_g4_p32", Workload("sp", 1, 40, 1500, 8, 2, 128, "bf16", seed=613), 32),
    ("decode_p1", Workload("s1", 1, 1, 900, 16, 4, 128, "bf16", k_global=200, window=32,
                           seed=614), 1),
]


@pytest.mark.parametrize("name,wl,P", SPARSE_CASES, ids=[c[0] for c in SPARSE_CASES])
def test_paged_sparse_token_equals_contiguous(name, wl, P):
    say(f"[paged sparse token] {name} {wl} page {P}")
    x = make_inputs(wl, device="cuda", n_sparse=1)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    _, lse = hs().full_attn_fwd(q, k, v)
    idx, cnt = hs().oracle_topk(q, k, lse, wl.k_global, wl.window) \
        if wl.n_q_heads // wl.n_kv_heads in (4, 8, 16) else (None, None)
    kp, table = paged(k, P, wl.seed)
    vp, _ = paged(v, P, wl.seed)
    g = torch.Generator().manual_seed(wl.seed)
    sink = torch.randn(wl.n_q_heads, generator=g).cuda()
    o, l1 = hs().sparse_attn_gather(qs, k, v, idx, cnt, kind="token", out_dtype=torch.float32,
                                    want_lse=True, sink=sink)
    o2, l2 = hs().sparse_attn_gather(qs, kp, vp, idx, cnt, kind="token", out_dtype=torch.float32,
                                     want_lse=True, sink=sink, pages=(table, wl.kv_len))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(l1, l2)
    # the paged layer against the oracle on the logical cache, with the same index sets
    r_o, r_l = oracle.masked_attention(to_numpy_f32(qs), to_numpy_f32(k), to_numpy_f32(v),
                                       idx.cpu().numpy(), cnt.cpu().numpy(),
                                       sink=sink.cpu().numpy())
    eo, el = max_abs(o2.cpu().numpy(), r_o), max_abs(l2.cpu().numpy(), r_l)
    say(f"  paged token layer with sinks vs oracle: max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
    assert eo <= TOL_BF16 and el <= LSE_TOL


GATED_CASES = [
    ("decode_g4_split_p64_ring", Workload("gd", 2, 1, 5000, 32, 8, 128, "bf16", block=64,
                                          n_blocks=16, window=128, seed=621), 64, 160),
    ("decode_g4_wide_p32", Workload("gw", 16, 1, 3000, 32, 8, 128, "bf16", block=64,
                                    n_blocks=16, window=128, seed=622), 32, 0),
    ("prefill_fused_p16_ring", Workload("gf", 1, 600, 1200, 16, 4, 128, "bf16", block=64,
                                        n_blocks=4, window=32, seed=623), 16, 700),
    ("prefill_split_p128", Workload("gp", 1, 70, 900, 8, 2, 128, "bf16", block=64, n_blocks=4,
                                    window=32, seed=624), 128, 0),
]


def ring_of(t, ring, first):
    """Position-indexed [B, T, Hkv, d] -> ring [B, ring, Hkv, d] holding positions >= first."""
    out = torch.zeros((t.shape[0], ring) + tuple(t.shape[2:]), dtype=t.dtype, device=t.device)
    for pos in range(first, t.shape[1]):
        out[:, pos % ring] = t[:, pos]
    return out


@pytest.mark.parametrize("name,wl,P,ring", GATED_CASES, ids=[c[0] for c in GATED_CASES])
def test_paged_gated_layer_equals_contiguous(name, wl, P, ring):
    say(f"[paged gated] {name} {wl} page {P} ring {ring}")
    x = make_inputs(wl, device="cuda", block_variant=True)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    _, lse = hs().full_attn_fwd(q, k, v)
    bi, bc = hs().block_score_topk(q, k, lse, wl.block, wl.n_blocks)
    kp, table = paged(k, P, wl.seed)
    vp, _ = paged(v, P, wl.seed)
    g = torch.Generator().manual_seed(wl.seed)
    s1, s2 = torch.randn(wl.n_q_heads, generator=g).cuda(), torch.randn(wl.n_q_heads, generator=g).cuda()
    swa = (x["k_loc"], x["v_loc"], x["gate"], wl.window)
    o, l1 = hs().sparse_attn_gather(qs, k, v, bi, bc, kind="block", block=wl.block, swa=swa,
                                    out_dtype=torch.float32, want_lse=True, sink=s1,
                                    sink_local=s2)
    if ring:
        first = wl.q_offset - wl.window + 1
        assert ring >= wl.window + wl.q_len - 1
        swa = (ring_of(x["k_loc"], ring, max(first, 0)), ring_of(x["v_loc"], ring, max(first, 0)),
               x["gate"], wl.window)
    o2, l2 = hs().sparse_attn_gather(qs, kp, vp, bi, bc, kind="block", block=wl.block, swa=swa,
                                     out_dtype=torch.float32, want_lse=True, sink=s1,
                                     sink_local=s2, local_ring=ring, pages=(table, wl.kv_len))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(l1, l2)
    # the paged (and ring) layer against the oracle on the logical, position-indexed caches,
    # with the same block sets and both sinks
    r_o, _, _ = oracle.gated_block_swa(to_numpy_f32(qs), to_numpy_f32(k), to_numpy_f32(v),
                                       bi.cpu().numpy(), bc.cpu().numpy(), wl.block,
                                       to_numpy_f32(x["k_loc"]), to_numpy_f32(x["v_loc"]),
                                       wl.window, x["gate"].cpu().numpy(),
                                       sink=s1.cpu().numpy(), sink_loc=s2.cpu().numpy())
    eo = max_abs(o2.cpu().numpy(), r_o)
    say(f"  paged gated layer (ring {ring}) vs oracle: max|dO| = {eo:.3e}")
    assert eo <= TOL_BF16


def test_paged_decode_pipeline_matches_oracle():
    """Paged full attention keeping the logits -> token selection from the logits -> a paged
    sparse layer, against the oracle on the logical cache."""
    wl = Workload("pipe", 2, 1, 6000, 32, 8, 128, "bf16", needles=8, seed=631)
    x = make_inputs(wl, device="cuda", n_sparse=1)
    kp, table = paged(x["k"], 64, 632)
    vp, _ = paged(x["v"], 64, 632)
    _, lse, lg = hs().full_attn_fwd_paged(x["q"], kp, vp, table, wl.kv_len, logits=True)
    idx, cnt = hs().oracle_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.k_global,
                                            wl.window)
    o, _ = hs().sparse_attn_gather(x["q_sparse"][0], kp, vp, idx, cnt, kind="token",
                                   out_dtype=torch.float32, pages=(table, wl.kv_len))
    torch.cuda.synchronize()
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    _, lse_ref = oracle.full_attention(qn, kn, vn)
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    ex = check_token_sets(gi, gc, oi, oc, qn, kn, lse_ref, wl.k_global, wl.window, wl.q_offset)
    say(f"  near-tie differences excused: {ex}")
    # outputs are compared on identical index sets: the GPU's own (checked above against the
    # oracle's, up to excused near-ties), fed to the oracle's masked attention
    o_ref, _ = oracle.masked_attention(to_numpy_f32(x["q_sparse"][0]), kn, vn, gi, gc)
    eo = max_abs(o.cpu().numpy(), o_ref)
    say(f"  sparse layer max|dO| = {eo:.3e}")
    assert eo <= TOL_BF16
