"""GPU parity of hs_full_attn_block_topk: full attention and the block-level oracle index in one
call (one pass on the prefill kernel for blocks of 64 and at most 16 blocks; two passes
otherwise) against the CPU oracle.

O and LSE must equal hs_full_attn_fwd's bit for bit (the same arithmetic); block sets follow the
near-tie rule of parity_utils.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import LSE_TOL, TOL_BF16, TOL_F32, check_block_sets, max_abs

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(x):
    return x.cuda() if torch.is_tensor(x) else x


CASES = [
    # one pass: prefill kernel, blocks of 64, n_blocks <= 16
    ("fused_g4_n16", Workload("f4", 1, 300, 2000, 8, 2, 128, "bf16", block=64, n_blocks=16,
                              seed=301)),
    ("fused_g16_n16", Workload("f16", 1, 50, 4000, 32, 2, 128, "bf16", block=64, n_blocks=16,
                               seed=302)),
    ("fused_g8_d64_n7", Workload("f8", 2, 100, 3000, 16, 2, 64, "bf16", block=64, n_blocks=7,
                                 seed=303)),
    ("fused_g1_n5", Workload("f1", 1, 40, 1500, 4, 4, 128, "bf16", block=64, n_blocks=5,
                             seed=304)),
    ("fused_g2_n16", Workload("f2", 1, 70, 2500, 8, 4, 128, "bf16", block=64, n_blocks=16,
                              seed=305)),
    # causal from position 0: early queries have fewer causal blocks than n_blocks
    ("fused_g4_causal_n3", Workload("fc", 2, 700, 700, 8, 2, 128, "bf16", block=64, n_blocks=3,
                                    seed=306)),
    ("fused_g4_n1", Workload("fn1", 1, 130, 1700, 8, 2, 128, "bf16", block=64, n_blocks=1,
                             seed=307)),
    ("fused_g16_causal_ragged", Workload("fr", 1, 333, 333, 32, 2, 128, "bf16", block=64,
                                         n_blocks=16, seed=308)),
    # 32 heads per KV head: one query's rows fill a whole wave
    ("fused_g32_n8", Workload("f32g", 1, 20, 1500, 64, 2, 128, "bf16", block=64, n_blocks=8,
                              seed=309)),
    # two passes
    ("decode_g4_b64", Workload("d4", 2, 1, 9000, 32, 8, 128, "bf16", block=64, n_blocks=16,
                               seed=311)),
    ("prefill_g8_b32", Workload("p32", 1, 37, 2000, 16, 2, 64, "bf16", block=32, n_blocks=7,
                                seed=312)),
    ("prefill_g4_b64_40blocks", Workload("p40", 1, 70, 3000, 8, 2, 128, "bf16", block=64,
                                         n_blocks=40, seed=313)),
    ("tiny_f32_b64", Workload("tf", 1, 200, 512, 4, 1, 64, "f32", block=64, n_blocks=4,
                              seed=314)),
]


@pytest.mark.parametrize("name,wl", CASES, ids=[c[0] for c in CASES])
def test_full_attn_block_topk_matches_oracle(name, wl):
    say(f"[full_attn_block_topk] {name} {wl}")
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o, lse, bi, bc = hs().full_attn_block_topk(q, k, v, wl.block, wl.n_blocks,
                                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    o2, lse2 = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "o / lse differ from full_attn_fwd"
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    o_ref, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    assert max_abs(o.cpu().numpy(), o_ref) <= (TOL_F32 if wl.dtype == "f32" else TOL_BF16)
    assert max_abs(lse.cpu().numpy(), lse_ref) <= LSE_TOL
    oi, oc = oracle.block_topk(qn, kn, lse_ref, wl.block, wl.n_blocks)
    excused = check_block_sets(bi.cpu().numpy(), bc.cpu().numpy(), oi, oc, qn, kn, lse_ref,
                               wl.block, wl.q_offset)
    say(f"  near-tie differences excused: {excused}")
    if wl.n_q_heads // wl.n_kv_heads in (4, 8, 16):  # the separate selection's group sizes
        b2, c2 = hs().block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        same = torch.equal(bi, b2) and torch.equal(bc, c2)
        say(f"  identical to the separate selection: {same}")


# Seeded sweep of the one-pass form: every group size it takes (1-32), both head sizes, ragged
# query counts, budgets 1-16, causal from position 0 and long prefixes.
#            g   hkv  d    Tq   Tk    n   b
SWEEP = [(1, 4, 128, 17, 900, 16, 1), (2, 2, 64, 61, 61, 3, 2), (4, 1, 128, 129, 2000, 1, 1),
         (8, 2, 64, 33, 1500, 13, 1), (16, 1, 128, 300, 300, 8, 1), (32, 1, 128, 4, 2100, 16, 2),
         (32, 2, 64, 9, 777, 5, 1), (16, 2, 64, 70, 3000, 16, 1), (8, 1, 128, 257, 257, 2, 1),
         (4, 4, 64, 100, 1100, 11, 2), (2, 1, 128, 200, 1600, 7, 1), (1, 2, 64, 40, 4000, 16, 1)]
SWEEP_CASES = [(f"sweep{i}_g{g}_hkv{h}_d{d}_tq{tq}_tk{tk}_n{n}_b{b}",
                Workload(f"fs{i}", b, tq, tk, g * h, h, d, "bf16", block=64, n_blocks=n,
                         seed=500 + i))
               for i, (g, h, d, tq, tk, n, b) in enumerate(SWEEP)]


@pytest.mark.parametrize("name,wl", SWEEP_CASES, ids=[c[0] for c in SWEEP_CASES])
def test_full_attn_block_topk_sweep(name, wl):
    test_full_attn_block_topk_matches_oracle(name, wl)


def test_fused_block_selection_keeps_lower_block_on_exact_ties():
    """Blocks whose maxima are exactly equal (copied key rows): the lower block ids win, as in
    the oracle, although the running list sees the tied blocks one tile at a time."""
    wl = Workload("ties", 1, 64, 3000, 8, 2, 128, "bf16", block=64, n_blocks=4, seed=321)
    x = make_inputs(wl)
    k = x["k"].clone()
    # one strong key for head 0 of KV head 0, copied into 6 blocks: 6 exactly equal block maxima
    qh = x["q"][0, -1, 0].float()
    k[0, 200, 0] = (8.0 * 128 ** 0.5 * qh / (qh * qh).sum()).to(k.dtype)
    for blk in (9, 12, 20, 25, 31):
        k[0, 64 * blk + 7, 0] = k[0, 200, 0]
    q_d, k_d, v_d = to_dev(x["q"]), to_dev(k), to_dev(x["v"])
    o, lse, bi, bc = hs().full_attn_block_topk(q_d, k_d, v_d, wl.block, wl.n_blocks)
    torch.cuda.synchronize()
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(k)
    _, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]))
    oi, oc = oracle.block_topk(qn, kn, lse_ref, wl.block, wl.n_blocks)
    assert np.array_equal(oi[0, -1, 0], [3, 9, 12, 20])
    assert np.array_equal(bi.cpu().numpy()[0, -1, 0], [3, 9, 12, 20])
    check_block_sets(bi.cpu().numpy(), bc.cpu().numpy(), oi, oc, qn, kn, lse_ref, wl.block,
                     wl.q_offset)
