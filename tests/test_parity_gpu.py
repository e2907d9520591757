"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Sizes here are ones the oracle finishes in seconds while still spanning many tiles, several
splits and ragged tails.  Index sets follow the near-tie rule of parity_utils; outputs are
compared with identical (oracle) index sets.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import (LSE_TOL, TOL_BF16, TOL_F32, check_block_sets, check_token_sets,
                          lse_bound, max_abs)

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(x):
    if isinstance(x, list):
        return [t.cuda() for t in x]
    return x.cuda() if torch.is_tensor(x) else x


# ---- full attention ----------------------------------------------------------------------

FULL_CASES = [
    # name, workload
    ("tiny_f32_prefill", Workload("tiny", 1, 512, 512, 4, 1, 64, "f32", seed=101)),
    ("decode_bf16_g4", Workload("dec", 2, 1, 5000, 32, 8, 128, "bf16", needles=4, seed=11)),
    ("decode_bf16_g16", Workload("dec16", 2, 1, 3001, 64, 4, 128, "bf16", seed=12)),
    ("short_block_bf16_d64", Workload("sb", 2, 3, 777, 8, 2, 64, "bf16", seed=13)),
    ("prefill_bf16_g4_ragged", Workload("pf", 1, 200, 1100, 8, 2, 128, "bf16", seed=14)),
    ("prefill_bf16_g16_chunk", Workload("pf16", 1, 77, 3000, 32, 2, 128, "bf16", seed=15)),
    ("prefill_bf16_g8_d64_causal", Workload("pf8", 2, 300, 300, 16, 2, 64, "bf16", seed=16)),
    ("prefill_bf16_g4_causal_long", Workload("pf4", 1, 700, 700, 8, 2, 128, "bf16", seed=17)),
    # group sizes outside the pages' models: 1 and 2 on the prefill kernel, 12 on the row kernel
    ("prefill_bf16_g1", Workload("pg1", 1, 300, 500, 4, 4, 128, "bf16", seed=18)),
    ("prefill_bf16_g2_d64", Workload("pg2", 2, 130, 400, 8, 4, 64, "bf16", seed=19)),
    ("prefill_bf16_g12", Workload("pg12", 1, 40, 600, 24, 2, 128, "bf16", seed=20)),
    # head size 256 with small groups: the 4-wave row kernel, also for prefill-shaped calls
    ("decode_bf16_g4_d256", Workload("d256", 2, 1, 3000, 8, 2, 256, "bf16", seed=21)),
    ("prefill_bf16_g8_d256", Workload("p256", 1, 30, 1200, 16, 2, 256, "bf16", seed=22)),
    ("prefill_bf16_g16_d256_causal", Workload("p256c", 1, 150, 150, 16, 1, 256, "bf16",
                                              seed=23)),
]


@pytest.mark.parametrize("name,wl", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_full_attn_matches_oracle(name, wl):
    say(f"[full_attn] {name} {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o, lse = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full_attention(to_numpy_f32(x["q"]), to_numpy_f32(x["k"]),
                                           to_numpy_f32(x["v"]))
    tol = TOL_F32 if wl.dtype == "f32" else TOL_BF16
    eo = max_abs(o.cpu().numpy(), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    say(f"  max|dO| = {eo:.3e}  max|dLSE| = {el:.3e}")
    assert eo <= tol
    assert el <= LSE_TOL
    # bf16 output path: within max(1e-2, one bf16 ulp) of the rounded oracle
    if wl.dtype == "bf16":
        ob, _ = hs().full_attn_fwd(q, k, v)
        ref_b = torch.from_numpy(o_ref).to(torch.bfloat16).float().numpy()
        diff = np.abs(ob.float().cpu().numpy() - ref_b)
        ulp = np.abs(ref_b) * 2.0 ** -7
        assert (diff <= np.maximum(TOL_BF16, ulp)).all()


def logit_profile_inputs(wl, profile):
    """Every query of a KV group is the same vector q0 and key i is s_i * sqrt(d) * q0 / |q0|^2,
    so every head sees the logit s_i at key i (up to bf16 rounding of the key)."""
    x = make_inputs(wl)
    q, k = x["q"].clone(), x["k"].clone()
    g = wl.n_q_heads // wl.n_kv_heads
    s = torch.tensor([profile(i) for i in range(wl.kv_len)], dtype=torch.float64)
    for b in range(wl.batch):
        for u in range(wl.n_kv_heads):
            q0 = q[b, 0, u * g].double()
            q[b, :, u * g:(u + 1) * g] = q0.to(q.dtype)
            dirv = wl.head_dim ** 0.5 * q0 / (q0 * q0).sum()
            k[b, :, u] = (s[:, None] * dirv[None, :]).to(k.dtype)
    return q, k, x["v"]


PROFILES = {
    # the maximum rises by about 32 log2 units along a row: the exponent reference of the
    # prefill kernel is kept while it is within 8 of the maximum and moved several times
    "linear_rise": lambda i: -8.0 + 22.0 * i / 2500,
    # one jump of 20 after a long flat stretch
    "step": lambda i: -8.0 if i < 1000 else 12.0,
    # rises and falls: late keys far below the reference
    "tent": lambda i: 14.0 - abs(i - 1200) * 0.02,
}


@pytest.mark.parametrize("profile", list(PROFILES), ids=list(PROFILES))
def test_full_attn_moving_maximum(profile):
    wl = Workload("mv", 1, 300, 2500, 8, 2, 128, "bf16", seed=41)
    say(f"[full_attn moving maximum] {profile} {wl}")
    q, k, v = logit_profile_inputs(wl, PROFILES[profile])
    o, lse = hs().full_attn_fwd(to_dev(q), to_dev(k), to_dev(v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full_attention(to_numpy_f32(q), to_numpy_f32(k), to_numpy_f32(v))
    eo = max_abs(o.cpu().numpy(), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    say(f"  max|dO| = {eo:.3e}  max|dLSE| = {el:.3e}  max LSE {np.abs(lse_ref).max():.2f}")
    assert eo <= TOL_BF16
    assert el <= lse_bound(lse_ref)


@pytest.mark.parametrize("profile", list(PROFILES), ids=list(PROFILES))
def test_full_attn_moving_maximum_row_kernel(profile):
    """The same logit profiles on decode shapes (one and three queries, split key ranges): the
    row kernel's online softmax and the split combine under a moving maximum."""
    for wl in (Workload("mvd", 2, 1, 2500, 8, 2, 128, "bf16", seed=42),
               Workload("mvd3", 1, 3, 2500, 16, 4, 64, "bf16", seed=43)):
        say(f"[full_attn moving maximum, row kernel] {profile} {wl}")
        q, k, v = logit_profile_inputs(wl, PROFILES[profile])
        o, lse = hs().full_attn_fwd(to_dev(q), to_dev(k), to_dev(v), out_dtype=torch.float32)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.full_attention(to_numpy_f32(q), to_numpy_f32(k), to_numpy_f32(v))
        eo = max_abs(o.cpu().numpy(), o_ref)
        el = max_abs(lse.cpu().numpy(), lse_ref)
        say(f"  max|dO| = {eo:.3e}  max|dLSE| = {el:.3e}")
        assert eo <= TOL_BF16
        assert el <= lse_bound(lse_ref)


# ---- token top-k -------------------------------------------------------------------------

TOPK_CASES = [
    ("tiny_f32_prefill", Workload("tiny", 1, 512, 512, 4, 1, 64, "f32", k_global=64, window=16,
                                  seed=101)),
    ("decode_g4_needles", Workload("dec", 2, 1, 9000, 32, 8, 128, "bf16", k_global=1024,
                                   window=128, needles=16, seed=21)),
    ("decode_g16_short", Workload("dec16", 1, 1, 1500, 64, 4, 128, "bf16", k_global=1024,
                                  window=128, seed=22)),
    ("decode_g8_two_queries", Workload("g8", 2, 2, 4000, 16, 2, 64, "bf16", k_global=100,
                                       window=20, seed=23)),
    ("prefill_g4_cross_cap", Workload("pfx", 1, 48, 1200, 8, 2, 128, "bf16", k_global=1024,
                                      window=128, seed=24)),
    # prefill selection: more than 2048 candidates per query forces buffer compactions
    ("prefill_g16_compactions", Workload("pfc", 1, 40, 6000, 32, 2, 128, "bf16",
                                         k_global=1024, window=128, seed=25)),
    ("prefill_g8_d64_small_k", Workload("pf8", 2, 100, 3000, 16, 2, 64, "bf16", k_global=50,
                                        window=10, seed=26)),
    # one workgroup per row over 3 and 4 key tiles of 32768 (ragged last tiles), and past
    # 131072 keys the multi-kernel boundary-list selection
    ("decode_g4_70k", Workload("dl", 1, 1, 70000, 32, 8, 128, "bf16", k_global=300, window=64,
                               needles=8, seed=27)),
    ("decode_g4_131k", Workload("d4t", 1, 1, 131072, 8, 2, 128, "bf16", k_global=1024,
                                window=128, needles=8, seed=31)),
    ("decode_g4_140k_chain", Workload("dch", 1, 1, 140000, 8, 2, 128, "bf16", k_global=1024,
                                      window=128, needles=8, seed=32)),
    # fewer candidates than k: every candidate is taken
    ("decode_g4_all_candidates", Workload("dall", 2, 1, 1000, 16, 4, 128, "bf16", k_global=1024,
                                          window=128, seed=33)),
    # decode rows with no candidates: window only (k_global = 0), and a context shorter than
    # the window
    ("decode_g4_window_only", Workload("dwo", 2, 1, 3000, 16, 4, 128, "bf16", k_global=0,
                                       window=40, seed=34)),
    ("decode_g4_short_context", Workload("dsc", 1, 1, 100, 8, 2, 128, "bf16", k_global=1024,
                                         window=128, seed=35)),
    # degenerate budgets: no forced window; window only (k_global = 0)
    ("decode_g4_no_window", Workload("dnw", 2, 1, 3000, 16, 4, 128, "bf16", k_global=200,
                                     window=0, seed=28)),
    ("prefill_g4_no_window", Workload("pnw", 1, 60, 900, 8, 2, 128, "bf16", k_global=100,
                                      window=0, seed=29)),
    ("prefill_g8_window_only", Workload("pwo", 1, 50, 700, 16, 2, 64, "bf16", k_global=0,
                                        window=40, seed=30)),
]


@pytest.mark.parametrize("name,wl", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_oracle_topk_matches_oracle(name, wl):
    say(f"[topk] {name} {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    _, lse = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
    idx, cnt = hs().oracle_topk(q, k, lse, wl.k_global, wl.window)
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


def _decode_sweep_cases():
    """Seeded decode shapes for the token selection: contexts from a few hundred keys to past
    131072 (one to five 32768-key tiles, ragged, and the tile edges themselves), every group
    size of the decode path, budgets from 0 to past the candidate count, windows 0 to 128."""
    tks = [300, 32768, 32769, 32896, 65536 + 3, 98304, 131072, 131200, 5000, 20000, 77777, 1200]
    ks = [2000, 1024, 17, 1, 256, 1024, 1024, 1024, 2000, 300, 0, 64]
    ws = [0, 128, 1, 64, 1, 128, 128, 0, 64, 1, 128, 128]
    cases = []
    for i, tk in enumerate(tks):
        g = [4, 8, 16][i % 3]
        hkv = [1, 2, 4][(i // 3) % 3]
        tq = 2 if g <= 8 and i % 2 else 1
        d = 64 if i % 4 == 3 else 128
        k, w = ks[i], ws[i]
        b = 1 + i % 3
        name = f"sweep{i}_b{b}_tq{tq}_tk{tk}_g{g}_hkv{hkv}_d{d}_k{k}_w{w}"
        cases.append((name, Workload(f"sw{i}", b, tq, tk, g * hkv, hkv, d, "bf16", k_global=k,
                                     window=w, seed=400 + i)))
    return cases


SWEEP_CASES = _decode_sweep_cases()


@pytest.mark.parametrize("name,wl", SWEEP_CASES, ids=[c[0] for c in SWEEP_CASES])
def test_decode_token_selection_sweep(name, wl):
    say(f"[topk sweep] {name}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    _, lse = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
    idx, cnt = hs().oracle_topk(q, k, lse, wl.k_global, wl.window)
    torch.cuda.synchronize()
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    excused = check_token_sets(idx.cpu().numpy(), cnt.cpu().numpy(), oi, oc, qn, kn, lse_ref,
                               wl.k_global, wl.window, wl.q_offset)
    say(f"  near-tie differences excused: {excused}")


def test_decode_selection_ties_across_key_tiles():
    """Exact ties spread over three 32768-key tiles of one decode row: the lowest positions win,
    so the cut falls inside the second tile after all of the first tile's copies."""
    wl = Workload("tiet", 1, 1, 70000, 8, 2, 128, "bf16", k_global=100, window=64, seed=62)
    say("[topk ties across tiles]")
    x = make_inputs(wl)
    k = x["k"].clone()
    qh = x["q"][0, -1, 0].float()
    needle = (8.0 * 128 ** 0.5 * qh / (qh * qh).sum()).to(k.dtype)
    copies = list(range(32700, 32820)) + list(range(65600, 65631))  # 68 + 52 + 31 copies
    k[0, copies, 0] = needle
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(k)
    q_d, k_d, v_d = to_dev(x["q"]), to_dev(k), to_dev(x["v"])
    _, lse = hs().full_attn_fwd(q_d, k_d, v_d)
    idx, cnt = hs().oracle_topk(q_d, k_d, lse, wl.k_global, wl.window)
    torch.cuda.synchronize()
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    want = np.array(copies[:100])
    assert np.array_equal(oi[0, 0, 0, :100], want)
    assert np.array_equal(gi[0, 0, 0, :100], want)
    excused = check_token_sets(gi, gc, oi, oc, qn, kn, lse_ref, wl.k_global, wl.window,
                               wl.q_offset)
    say(f"  near-tie differences excused: {excused}")


@pytest.mark.parametrize("q_len", [1, 33])
def test_token_selection_exact_ties_prefer_lower_position(q_len):
    """Exactly equal scores: both selection paths (few and many query rows) must keep the lower
    positions, as the oracle does."""
    wl = Workload("ties", 1, q_len, 3000, 8, 2, 128, "bf16", k_global=50, window=16, seed=61)
    say(f"[topk ties] q_len={q_len}")
    x = make_inputs(wl)
    k = x["k"].clone()
    # one needle for head 0 of KV head 0 copied to 81 positions (500, 1000..1079): each copy gets
    # p ~ 1/81, above every other key of the group, so the 50 selected candidates are all copies
    # and the tie rule alone decides which (the lowest positions)
    qh = x["q"][0, -1, 0].float()
    k[0, 500, 0] = (8.0 * 128 ** 0.5 * qh / (qh * qh).sum()).to(k.dtype)
    k[0, 1000:1080, 0] = k[0, 500, 0]
    k[0, 100:700, 1] = k[0, 1000:1600, 1]  # scattered ties for KV head 1
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(k)
    q_d, k_d, v_d = to_dev(x["q"]), to_dev(k), to_dev(x["v"])
    _, lse = hs().full_attn_fwd(q_d, k_d, v_d)
    idx, cnt = hs().oracle_topk(q_d, k_d, lse, wl.k_global, wl.window)
    torch.cuda.synchronize()
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    want = np.array([500] + list(range(1000, 1049)))
    assert np.array_equal(oi[0, -1, 0, :50], want)
    assert np.array_equal(gi[0, -1, 0, :50], want)
    excused = check_token_sets(gi, gc, oi, oc, qn, kn, lse_ref, wl.k_global, wl.window,
                               wl.q_offset)
    say(f"  near-tie differences excused: {excused}")


# ---- block scores + top-n blocks ----------------------------------------------------------

BLOCK_CASES = [
    ("tiny_f32_b16", Workload("tb", 1, 512, 512, 4, 1, 64, "f32", block=16, n_blocks=5, seed=51)),
    ("decode_g4_b64", Workload("bd", 2, 1, 9000, 32, 8, 128, "bf16", block=64, n_blocks=16,
                               needles=8, seed=52)),
    ("decode_g16_b64", Workload("bd16", 1, 1, 4100, 64, 4, 128, "bf16", block=64, n_blocks=16,
                                seed=53)),
    ("prefill_g8_b32", Workload("bp", 1, 37, 2000, 16, 2, 64, "bf16", block=32, n_blocks=7,
                                seed=54)),
    ("prefill_g16_b64", Workload("bp16", 1, 50, 4000, 32, 2, 128, "bf16", block=64,
                                 n_blocks=16, seed=55)),
    ("prefill_g4_b64_causal", Workload("bp4", 2, 300, 300, 8, 2, 128, "bf16", block=64,
                                       n_blocks=3, seed=56)),
    ("prefill_g4_b128_generic", Workload("bpg", 1, 30, 1500, 8, 2, 128, "bf16", block=128,
                                         n_blocks=5, seed=57)),
    # more than 16 blocks per list (4 register entries per lane on the prefill path); the most
    ("prefill_g4_b32_40blocks", Workload("bp40", 1, 70, 3000, 8, 2, 128, "bf16", block=32,
                                         n_blocks=40, seed=58)),
    ("decode_g8_b64_64blocks", Workload("bd64", 2, 1, 6000, 32, 4, 128, "bf16", block=64,
                                        n_blocks=64, seed=59)),
    # blocks that are multiples of 16 but do not divide 64 (the generic path in both shapes)
    ("decode_g4_b48", Workload("b48", 2, 1, 5000, 16, 4, 128, "bf16", block=48, n_blocks=20,
                               seed=60)),
    ("prefill_g8_b80_generic", Workload("b80", 1, 25, 2000, 16, 2, 64, "bf16", block=80,
                                        n_blocks=9, seed=61)),
]


@pytest.mark.parametrize("name,wl", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_block_topk_matches_oracle(name, wl):
    say(f"[block topk] {name} {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    _, lse = hs().full_attn_fwd(q, k, v)
    bi, bc = hs().block_score_topk(q, k, lse, wl.block, wl.n_blocks)
    torch.cuda.synchronize()
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.block_topk(qn, kn, lse_ref, wl.block, wl.n_blocks)
    excused = check_block_sets(bi.cpu().numpy(), bc.cpu().numpy(), oi, oc, qn, kn, lse_ref,
                               wl.block, wl.q_offset)
    say(f"  near-tie differences excused: {excused}")


# ---- sparse attention over the oracle's index sets ----------------------------------------

SPARSE_CASES = [
    ("tiny_f32_token", Workload("tiny", 1, 512, 512, 4, 1, 64, "f32", k_global=64, window=16,
                                seed=101)),
    ("decode_g4_token", Workload("dec", 3, 1, 6000, 32, 8, 128, "bf16", needles=8, seed=31)),
    ("decode_g16_token", Workload("d16", 2, 1, 2500, 64, 4, 128, "bf16", seed=32)),
    ("prefill_g4_token", Workload("pf", 1, 40, 1500, 8, 2, 128, "bf16", seed=33)),
    # at least 96 (query, KV head) sets: one 8-wave workgroup per set, no split
    ("prefill_g4_token_wide", Workload("pw", 1, 120, 2000, 8, 2, 128, "bf16", seed=35)),
    ("decode_g4_token_wide", Workload("dw", 16, 1, 4000, 32, 8, 128, "bf16", seed=36)),
    ("decode_g8_d64_token_wide", Workload("dw64", 12, 1, 3000, 64, 8, 64, "bf16",
                                          k_global=500, window=64, seed=37)),
    ("decode_g1_token", Workload("dg1", 2, 1, 3000, 8, 8, 128, "bf16", seed=38)),
    ("prefill_g2_token", Workload("pg2", 1, 30, 1500, 4, 2, 128, "bf16", seed=39)),
    # head size 256 on the row kernel, and groups of 32 / 64 heads (the group kernel) with
    # several queries
    ("decode_g8_d256_token", Workload("d256", 2, 1, 2000, 16, 2, 256, "bf16", k_global=300,
                                      window=32, seed=40)),
    ("prefill_g4_d256_token", Workload("p256", 1, 20, 900, 8, 2, 256, "bf16", k_global=200,
                                       window=16, seed=41)),
    ("decode_g32_d128_token", Workload("d32", 2, 1, 2500, 64, 2, 128, "bf16", k_global=400,
                                       window=64, seed=42)),
    ("prefill_g64_d256_token", Workload("p64", 1, 5, 1000, 64, 1, 256, "bf16", k_global=300,
                                        window=32, seed=43)),
]


@pytest.mark.parametrize("name,wl", SPARSE_CASES, ids=[c[0] for c in SPARSE_CASES])
def test_sparse_token_matches_oracle(name, wl):
    say(f"[sparse token] {name} {wl}")
    x = make_inputs(wl, n_sparse=2)
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    oi, oc = oracle.token_topk(qn, kn, None, wl.k_global, wl.window)
    k, v = to_dev(x["k"]), to_dev(x["v"])
    idx = torch.from_numpy(oi).cuda()
    cnt = torch.from_numpy(oc).cuda()
    tol = TOL_F32 if wl.dtype == "f32" else TOL_BF16
    for layer, qs in enumerate(x["q_sparse"]):
        o, lse = hs().sparse_attn_gather(to_dev(qs), k, v, idx, cnt, kind="token",
                                         out_dtype=torch.float32, want_lse=True)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.masked_attention(to_numpy_f32(qs), kn, vn, oi, oc)
        eo, el = max_abs(o.cpu().numpy(), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
        say(f"  layer {layer}: max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
        assert eo <= tol and el <= LSE_TOL


def test_sparse_token_budget_covering_prefix_equals_full_attention():
    """k + w >= t + 1: the sparse layer must reproduce full attention with the same Q'."""
    wl = Workload("cov", 1, 64, 64, 8, 2, 128, "bf16", k_global=48, window=16, seed=34)
    say(f"[sparse cover] {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    qs = to_dev(x["q_sparse"][0])
    _, lse = hs().full_attn_fwd(q, k, v)
    idx, cnt = hs().oracle_topk(q, k, lse, wl.k_global, wl.window)
    o_s, _ = hs().sparse_attn_gather(qs, k, v, idx, cnt, out_dtype=torch.float32)
    o_f, _ = hs().full_attn_fwd(qs, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (cnt.cpu().numpy() == np.arange(1, wl.q_len + 1)[None, :, None]).all()
    # the two kernels sum in different orders (bf16 P), so the bar is the bf16 output tolerance
    o_ref, _ = oracle.full_attention(to_numpy_f32(x["q_sparse"][0]), to_numpy_f32(x["k"]),
                                     to_numpy_f32(x["v"]))
    assert max_abs(o_s.cpu().numpy(), o_ref) <= TOL_BF16
    assert max_abs(o_f.cpu().numpy(), o_ref) <= TOL_BF16
    assert max_abs(o_s.cpu().numpy(), o_f.cpu().numpy()) <= TOL_BF16


GATED_CASES = [
    ("decode_g4", Workload("gd", 2, 1, 5000, 32, 8, 128, "bf16", block=64, n_blocks=16,
                           window=128, seed=41)),
    ("prefill_g4_ragged", Workload("gp", 1, 70, 900, 8, 2, 128, "bf16", block=64, n_blocks=4,
                                   window=32, seed=42)),
    ("tiny_f32", Workload("gt", 1, 128, 512, 4, 1, 64, "f32", block=16, n_blocks=5, window=16,
                          seed=43)),
    # at least 2048 (query, KV head) sets: both branches unsplit, run in one workgroup
    ("prefill_fused_g4", Workload("gf", 1, 600, 1200, 16, 4, 128, "bf16", block=64, n_blocks=4,
                                  window=32, seed=44)),
    ("prefill_fused_f32_d64", Workload("gf32", 1, 520, 600, 16, 4, 64, "f32", block=16,
                                       n_blocks=6, window=20, seed=45)),
    # other group and head sizes: 16, 8 with d 64 and blocks of 32, d 256 (two branches and a
    # combine), and a 32-head group with two queries
    ("decode_g16", Workload("g16", 2, 1, 3000, 64, 4, 128, "bf16", block=64, n_blocks=16,
                            window=64, seed=46)),
    ("decode_g8_d64_b32", Workload("g8", 3, 1, 2500, 16, 2, 64, "bf16", block=32, n_blocks=12,
                                   window=48, seed=47)),
    ("decode_g4_d256", Workload("g256", 2, 1, 2000, 8, 2, 256, "bf16", block=64, n_blocks=8,
                                window=64, seed=48)),
    ("g32_two_queries", Workload("g32", 1, 2, 2000, 64, 2, 128, "bf16", block=64, n_blocks=8,
                                 window=64, seed=49)),
]


@pytest.mark.parametrize("name,wl", GATED_CASES, ids=[c[0] for c in GATED_CASES])
def test_block_sparse_gated_swa_matches_oracle(name, wl):
    say(f"[block+swa] {name} {wl}")
    x = make_inputs(wl, block_variant=True)
    a = {n: to_numpy_f32(x[n]) for n in ("q", "k", "v", "k_loc", "v_loc", "gate")}
    qs = x["q_sparse"][0]
    bi, bc = oracle.block_topk(a["q"], a["k"], None, wl.block, wl.n_blocks)
    o_ref, _, _ = oracle.gated_block_swa(to_numpy_f32(qs), a["k"], a["v"], bi, bc, wl.block,
                                         a["k_loc"], a["v_loc"], wl.window, a["gate"])
    o, _ = hs().sparse_attn_gather(
        to_dev(qs), to_dev(x["k"]), to_dev(x["v"]), torch.from_numpy(bi).cuda(),
        torch.from_numpy(bc).cuda(), kind="block", block=wl.block,
        swa=(to_dev(x["k_loc"]), to_dev(x["v_loc"]), to_dev(x["gate"]), wl.window),
        out_dtype=torch.float32)
    torch.cuda.synchronize()
    tol = TOL_F32 if wl.dtype == "f32" else TOL_BF16
    eo = max_abs(o.cpu().numpy(), o_ref)
    say(f"  max|dO| = {eo:.3e}")
    assert eo <= tol


def test_sparse_token_empty_index_sets():
    """Sets with count 0 attend over nothing: output 0 and LSE -inf; the other sets as usual."""
    wl = Workload("emp", 2, 3, 1200, 8, 2, 128, "bf16", k_global=64, window=16, seed=60)
    say(f"[sparse empty sets] {wl}")
    x = make_inputs(wl)
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    oi, oc = oracle.token_topk(qn, kn, None, wl.k_global, wl.window)
    empty = np.zeros_like(oc, dtype=bool)
    empty[1, 2, 0] = empty[0, 0, 1] = True
    oc_gpu = oc.copy()
    oc_gpu[empty] = 0
    qs = x["q_sparse"][0]
    o, lse = hs().sparse_attn_gather(to_dev(qs), to_dev(x["k"]), to_dev(x["v"]),
                                     torch.from_numpy(oi).cuda(), torch.from_numpy(oc_gpu).cuda(),
                                     kind="token", out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    o_ref, lse_ref = oracle.masked_attention(to_numpy_f32(qs), kn, vn, oi, oc)
    g = wl.group
    for b in range(wl.batch):
        for j in range(wl.q_len):
            for u in range(wl.n_kv_heads):
                hs_ = slice(u * g, (u + 1) * g)
                if empty[b, j, u]:
                    assert (o[b, j, hs_] == 0).all()
                    assert np.isneginf(lse[b, hs_, j]).all()
                else:
                    assert max_abs(o[b, j, hs_], o_ref[b, j, hs_]) <= TOL_BF16
                    assert max_abs(lse[b, hs_, j], lse_ref[b, hs_, j]) <= LSE_TOL



# ---- a logit scale other than 1/sqrt(d) ------------------------------------------------------

SCALE_CASES = [
    ("decode_g4", Workload("sc_dec", 2, 1, 4000, 32, 8, 128, "bf16", k_global=256, window=64,
                           block=64, n_blocks=8, seed=131), 0.0625),
    ("prefill_g8_ragged", Workload("sc_pf", 1, 150, 900, 16, 2, 128, "bf16", k_global=128,
                                   window=32, block=64, n_blocks=4, seed=132), 0.11),
    ("tiny_f32", Workload("sc_t", 1, 64, 200, 4, 1, 64, "f32", k_global=32, window=8, block=16,
                          n_blocks=4, seed=133), 0.09),
]


@pytest.mark.parametrize("name,wl,scale", SCALE_CASES, ids=[c[0] for c in SCALE_CASES])
def test_scale_is_applied_everywhere(name, wl, scale):
    """desc.scale replaces 1/sqrt(d) in every call of a hybrid block: full attention, token and
    block selection, token-sparse and gated block-sparse layers, against the oracle with the same
    scale (outputs on the oracle's index sets)."""
    say(f"[scale {scale}] {name} {wl}")
    x = make_inputs(wl, block_variant=True)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    qs = to_dev(x["q_sparse"][0])
    o, lse = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32, scale=scale)
    idx, cnt = hs().oracle_topk(q, k, lse, wl.k_global, wl.window, scale=scale)
    bidx, bcnt = hs().block_score_topk(q, k, lse, wl.block, wl.n_blocks, scale=scale)
    torch.cuda.synchronize()
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.full_attention(qn, kn, vn, scale=scale)
    eo, el = max_abs(o.cpu().numpy(), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    say(f"  full attention max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
    tol = TOL_F32 if wl.dtype == "f32" else TOL_BF16
    assert eo <= tol and el <= LSE_TOL
    # the default scale gives different logits: the check above is not vacuous
    _, lse_def = oracle.full_attention(qn, kn, vn)
    assert max_abs(lse_def, lse_ref) > 1e-2
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window, scale=scale)
    ex = 0
    for b in range(wl.batch):
        for j in range(wl.q_len):
            for u in range(wl.n_kv_heads):
                n = int(oc[b, j, u])
                assert int(cnt[b, j, u]) == n
                gs, os_ = idx[b, j, u, :n].cpu().numpy(), oi[b, j, u, :n]
                if not np.array_equal(gs, os_):
                    s = oracle.token_score_row(qn, kn, lse_ref, b, j, u, scale=scale)
                    sel = os_[os_ < wl.q_offset + j - wl.window + 1]
                    s_k = s[sel].min()
                    d = np.setxor1d(gs, os_)
                    assert (np.abs(s[d] - s_k) <= 1e-6 * s_k).all(), (b, j, u)
                    ex += len(d)
    bi, bc = oracle.block_topk(qn, kn, lse_ref, wl.block, wl.n_blocks, scale=scale)
    for b in range(wl.batch):
        for j in range(wl.q_len):
            for u in range(wl.n_kv_heads):
                n = int(bc[b, j, u])
                assert int(bcnt[b, j, u]) == n
                gs, os_ = bidx[b, j, u, :n].cpu().numpy(), bi[b, j, u, :n]
                if not np.array_equal(gs, os_):
                    s = oracle.block_score_row(qn, kn, lse_ref, b, j, u, wl.block, scale=scale)
                    d = np.setxor1d(gs, os_)
                    assert (np.abs(s[d] - s[os_].min()) <= 1e-6 * s[os_].min()).all(), (b, j, u)
                    ex += len(d)
    say(f"  index sets: near-tie differences excused {ex}")
    so, _ = hs().sparse_attn_gather(qs, k, v, to_dev(torch.from_numpy(oi)),
                                    to_dev(torch.from_numpy(oc)), out_dtype=torch.float32,
                                    scale=scale)
    swa = (to_dev(x["k_loc"]), to_dev(x["v_loc"]), to_dev(x["gate"]), wl.window)
    go, _ = hs().sparse_attn_gather(qs, k, v, to_dev(torch.from_numpy(bi)),
                                    to_dev(torch.from_numpy(bc)), kind="block", block=wl.block,
                                    swa=swa, out_dtype=torch.float32, scale=scale)
    torch.cuda.synchronize()
    qsn = to_numpy_f32(x["q_sparse"][0])
    so_ref, _ = oracle.masked_attention(qsn, kn, vn, oi, oc, scale=scale)
    go_ref, _, _ = oracle.gated_block_swa(qsn, kn, vn, bi, bc, wl.block,
                                          to_numpy_f32(x["k_loc"]), to_numpy_f32(x["v_loc"]),
                                          wl.window, x["gate"].numpy(), scale=scale)
    es, eg = max_abs(so.cpu().numpy(), so_ref), max_abs(go.cpu().numpy(), go_ref)
    say(f"  token-sparse max|dO| = {es:.3e}  gated block layer max|dO| = {eg:.3e}")
    assert es <= tol and eg <= tol


@pytest.mark.parametrize("profile", ["step", "linear_rise"])
def test_full_attn_d256_prefill_moving_maximum(profile):
    """Head size 256 on the tiled prefill kernel (128 rows per workgroup, 32-key tiles) with a
    row maximum that moves by more than the lazy-rescale margin."""
    wl = Workload("mv256", 1, 96, 2500, 16, 2, 256, "bf16", seed=43)
    say(f"[full_attn d256 moving maximum] {profile} {wl}")
    q, k, v = logit_profile_inputs(wl, PROFILES[profile])
    o, lse = hs().full_attn_fwd(to_dev(q), to_dev(k), to_dev(v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full_attention(to_numpy_f32(q), to_numpy_f32(k), to_numpy_f32(v))
    eo = max_abs(o.cpu().numpy(), o_ref)
    el = max_abs(lse.cpu().numpy(), lse_ref)
    say(f"  max|dO| = {eo:.3e}  max|dLSE| = {el:.3e}")
    assert eo <= TOL_BF16
    assert el <= lse_bound(lse_ref)
