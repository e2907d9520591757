"""GPU parity of the decode path that keeps the full-attention logits: hs_full_attn_fwd_logits,
hs_oracle_topk_from_logits and hs_block_topk_from_logits against the CPU oracle.

The stored logits are compared with the oracle's a = q.k / sqrt(d) within the rounding bound of
an fp32 dot product of d terms; the index sets follow the near-tie rule of parity_utils (they
are the oracle's own sets up to ties that fp32 may resolve either way).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import LSE_TOL, check_block_sets, check_token_sets

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(x):
    return x.cuda() if torch.is_tensor(x) else x


def row_kernel_route(wl):
    """hs_full_attn_fwd runs the kernel that can keep logits (the row kernel, or the group kernel
    for groups of more than 16 heads) for these shapes, i.e. not the prefill kernel."""
    g = wl.n_q_heads // wl.n_kv_heads
    rows = wl.q_len * g
    prefill = (wl.dtype != "f32" and wl.head_dim <= 128 and rows > 16
               and (g <= 16 or rows >= 128) and 256 % g == 0)
    return not prefill


LOGIT_CASES = [
    ("decode_g4", Workload("dec", 2, 1, 5000, 32, 8, 128, "bf16", needles=4, seed=201)),
    # kv_len not a multiple of 4: scalar stores of the logits
    ("decode_g16_ragged", Workload("d16", 2, 1, 3001, 64, 4, 128, "bf16", seed=202)),
    ("short_block_d64", Workload("sb", 2, 3, 777, 8, 2, 64, "bf16", seed=203)),
    ("decode_g1", Workload("g1", 1, 1, 2000, 8, 8, 128, "bf16", seed=204)),
    ("decode_g12", Workload("g12", 1, 1, 1999, 24, 2, 128, "bf16", seed=205)),
    ("tiny_f32_prefill", Workload("tiny", 1, 64, 300, 4, 1, 64, "f32", seed=206)),
    ("one_key", Workload("one", 1, 1, 1, 8, 2, 128, "bf16", seed=207)),
    # groups of more than 16 heads (the group kernel): MQA d 256, an odd key count; 48 heads
    # (three chunks) with two queries; 32 heads on two KV heads
    ("mqa64_d256_odd", Workload("m", 1, 1, 2999, 64, 1, 256, "bf16", seed=208)),
    ("g48_d128_two_queries", Workload("g48", 1, 2, 2001, 48, 1, 128, "bf16", seed=209)),
    ("g32_d256_two_kv_heads", Workload("g32", 2, 1, 4000, 64, 2, 256, "bf16", seed=210)),
]


@pytest.mark.parametrize("name,wl", LOGIT_CASES, ids=[c[0] for c in LOGIT_CASES])
def test_full_attn_logits_match_oracle(name, wl):
    say(f"[full_attn_logits] {name} {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o, lse, lg = hs().full_attn_fwd_logits(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    if row_kernel_route(wl):
        o2, lse2 = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
        assert torch.equal(o, o2) and torch.equal(lse, lse2), "outputs differ from full_attn_fwd"
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    o_ref, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    tol = 1e-5 if wl.dtype == "f32" else 1e-2
    assert float(np.max(np.abs(o.cpu().numpy() - o_ref))) <= tol
    assert float(np.max(np.abs(lse.cpu().numpy() - lse_ref))) <= LSE_TOL
    d = wl.head_dim
    tau = 1.0 / math.sqrt(d)
    lgn = lg.cpu().numpy().astype(np.float64)
    worst = 0.0
    js = range(wl.q_len) if wl.q_len <= 4 else (0, 1, wl.q_len // 2, wl.q_len - 1)
    for b in range(wl.batch):
        for j in js:
            t = wl.q_offset + j
            for h in range(wl.n_q_heads):
                u = h // (wl.n_q_heads // wl.n_kv_heads)
                a = oracle.logit_row(qn, kn, b, j, h)
                # fp32 sum of d exact (bf16) or rounded (fp32) products: |err| <= (d+1) u sum|q k|
                mag = np.abs(kn[b, :t + 1, u].astype(np.float64)) @ np.abs(qn[b, j, h].astype(np.float64))
                bound = tau * (d + 1) * 2.0 ** -24 * mag + 1e-30
                err = np.abs(lgn[b, j, h, :t + 1] * tau - a)
                assert (err <= bound).all(), (b, j, h, int(np.argmax(err - bound)))
                worst = max(worst, float(np.max(err / bound)))
    say(f"  logits within {worst:.3f} of the fp32 rounding bound")


TOPK_CASES = [
    ("decode_g4_needles", Workload("dec", 2, 1, 9000, 32, 8, 128, "bf16", k_global=1024,
                                   window=128, needles=16, seed=211)),
    ("decode_g16_short", Workload("dec16", 1, 1, 1500, 64, 4, 128, "bf16", k_global=1024,
                                  window=128, seed=212)),
    ("decode_g8_two_queries", Workload("g8", 2, 2, 4001, 16, 2, 64, "bf16", k_global=100,
                                       window=20, seed=213)),
    ("decode_g1", Workload("g1", 1, 1, 3000, 8, 8, 128, "bf16", k_global=200, window=32,
                           seed=214)),
    ("decode_g2_three_queries", Workload("g2", 1, 3, 2500, 8, 4, 128, "bf16", k_global=300,
                                         window=16, seed=215)),
    ("decode_g12", Workload("g12", 1, 1, 2999, 24, 2, 128, "bf16", k_global=256, window=64,
                            seed=216)),
    ("decode_g4_70k", Workload("dl", 1, 1, 70000, 32, 8, 128, "bf16", k_global=300, window=64,
                               needles=8, seed=217)),
    ("decode_g4_no_window", Workload("dnw", 2, 1, 3000, 16, 4, 128, "bf16", k_global=200,
                                     window=0, seed=218)),
    ("decode_g4_window_only", Workload("dwo", 1, 1, 900, 16, 4, 128, "bf16", k_global=0,
                                       window=40, seed=219)),
    # fewer keys than the forced window: no candidates at all
    ("decode_short_context", Workload("dsc", 2, 1, 100, 16, 4, 128, "bf16", k_global=1024,
                                      window=128, seed=220)),
    ("tiny_f32_prefill", Workload("tiny", 1, 40, 512, 4, 1, 64, "f32", k_global=64, window=16,
                                  seed=221)),
]


@pytest.mark.parametrize("name,wl", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_from_logits_matches_oracle(name, wl):
    say(f"[topk_from_logits] {name} {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    _, lse, lg = hs().full_attn_fwd_logits(q, k, v)
    idx, cnt = hs().oracle_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.k_global,
                                            wl.window)
    torch.cuda.synchronize()
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    excused = check_token_sets(idx.cpu().numpy(), cnt.cpu().numpy(), oi, oc, qn, kn, lse_ref,
                               wl.k_global, wl.window, wl.q_offset)
    say(f"  near-tie differences excused: {excused}")
    if wl.needles:
        for b in range(wl.batch):
            for u in range(wl.n_kv_heads):
                sel = set(idx[b, -1, u, :cnt[b, -1, u]].cpu().tolist())
                assert set(x["needle_pos"][b, u].tolist()) <= sel
    g = wl.n_q_heads // wl.n_kv_heads
    if g in (4, 8, 16) and row_kernel_route(wl):
        i2, c2 = hs().oracle_topk(q, k, lse, wl.k_global, wl.window)
        same = torch.equal(idx, i2) and torch.equal(cnt, c2)
        say(f"  identical to the recomputing selection: {same}")


def test_topk_from_logits_exact_ties_prefer_lower_position():
    """Exactly equal scores: the lower positions are kept, as the oracle does (the inputs of
    the recomputing selection's tie test: with this seed the 50 candidates are all copies)."""
    wl = Workload("ties", 1, 1, 3000, 8, 2, 128, "bf16", k_global=50, window=16, seed=61)
    x = make_inputs(wl)
    k = x["k"].clone()
    qh = x["q"][0, -1, 0].float()
    k[0, 500, 0] = (8.0 * 128 ** 0.5 * qh / (qh * qh).sum()).to(k.dtype)
    k[0, 1000:1080, 0] = k[0, 500, 0]
    k[0, 100:700, 1] = k[0, 1000:1600, 1]
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(k)
    q_d, k_d, v_d = to_dev(x["q"]), to_dev(k), to_dev(x["v"])
    _, lse, lg = hs().full_attn_fwd_logits(q_d, k_d, v_d)
    idx, cnt = hs().oracle_topk_from_logits(lg, lse, 2, 128, wl.k_global, wl.window)
    torch.cuda.synchronize()
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    want = np.array([500] + list(range(1000, 1049)))
    assert np.array_equal(oi[0, -1, 0, :50], want)
    assert np.array_equal(gi[0, -1, 0, :50], want)
    check_token_sets(gi, gc, oi, oc, qn, kn, lse_ref, wl.k_global, wl.window, wl.q_offset)


BLOCK_CASES = [
    ("decode_g4_b64", Workload("bd", 2, 1, 9000, 32, 8, 128, "bf16", block=64, n_blocks=16,
                               needles=8, seed=241)),
    ("decode_g16_b64_ragged", Workload("bd16", 1, 1, 4101, 64, 4, 128, "bf16", block=64,
                                       n_blocks=16, seed=242)),
    ("decode_g8_b64_64blocks", Workload("bd64", 2, 1, 6000, 32, 4, 128, "bf16", block=64,
                                        n_blocks=64, seed=243)),
    ("decode_g2_b16_two_queries", Workload("b2", 1, 2, 3000, 8, 4, 64, "bf16", block=16,
                                           n_blocks=20, seed=244)),
    ("decode_g1_b128", Workload("b1", 2, 1, 5000, 4, 4, 128, "bf16", block=128, n_blocks=8,
                                seed=245)),
    # fewer causal blocks than n_blocks
    ("decode_short_b64", Workload("bs", 1, 1, 300, 16, 4, 128, "bf16", block=64, n_blocks=16,
                                  seed=246)),
    ("tiny_f32_b32", Workload("tb", 1, 30, 512, 4, 1, 64, "f32", block=32, n_blocks=5, seed=247)),
    # longer than 256 blocks per split at the geometry's cap: several splits merged
    ("decode_g4_b64_100k", Workload("bl", 1, 1, 100000, 32, 8, 128, "bf16", block=64,
                                    n_blocks=16, seed=248)),
]


@pytest.mark.parametrize("name,wl", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_block_topk_from_logits_matches_oracle(name, wl):
    say(f"[block_topk_from_logits] {name} {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    _, lse, lg = hs().full_attn_fwd_logits(q, k, v)
    bi, bc = hs().block_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.block,
                                         wl.n_blocks)
    torch.cuda.synchronize()
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.block_topk(qn, kn, lse_ref, wl.block, wl.n_blocks)
    excused = check_block_sets(bi.cpu().numpy(), bc.cpu().numpy(), oi, oc, qn, kn, lse_ref,
                               wl.block, wl.q_offset)
    say(f"  near-tie differences excused: {excused}")
    g = wl.n_q_heads // wl.n_kv_heads
    if g in (4, 8, 16) and row_kernel_route(wl):
        b2, c2 = hs().block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        say(f"  identical to the recomputing selection: {torch.equal(bi, b2) and torch.equal(bc, c2)}")
