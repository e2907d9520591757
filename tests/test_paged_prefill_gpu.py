"""GPU parity of prefill over a paged K / V cache: hs_full_attn_fwd_paged on the tiled prefill
kernel, hs_oracle_topk_paged and hs_block_score_topk_paged on the streamed prefill selection,
and a paged token-sparse layer over many queries.  The same logical cache laid out in shuffled
pages must give bit-identical outputs to the contiguous calls, and every output is compared with
the oracle on the logical cache (index sets bit-exact up to near-ties, outputs on identical sets
within the bf16 bound, LSE within 1e-6).  Prefill and decode over a paged cache take their own
kernels [P2 engineering constraints 2 and 3].
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import TOL_BF16, check_block_sets, check_token_sets, lse_bound, max_abs, paged

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (name, workload, page size): prefill shapes (many query rows per KV head), ragged key and
# query counts, pages of one tile and of several, head sizes 64, 128 and 256, groups of 4-64
CASES = [
    ("g4_d128_p64", Workload("pp4", 2, 200, 3001, 16, 4, 128, "bf16", k_global=256, window=64,
                             needles=6, seed=701), 64),
    ("g16_d128_p128", Workload("pp16", 1, 96, 5000, 32, 2, 128, "bf16", k_global=512,
                               window=128, needles=8, seed=702), 128),
    ("g8_d64_p256", Workload("pp8", 1, 130, 2100, 16, 2, 64, "bf16", k_global=128, window=32,
                             needles=4, seed=703), 256),
    ("mqa64_d256_p64", Workload("ppm", 1, 32, 3000, 64, 1, 256, "bf16", k_global=256,
                                window=64, needles=4, seed=704), 64),
    # two chunks of 16 heads and their exact merge; blocks of 32 keys
    ("g32_d128_p128_blk32", Workload("pp32", 1, 40, 4100, 64, 2, 128, "bf16", k_global=384,
                                     window=64, block=32, n_blocks=24, needles=6, seed=707), 128),
    # just past the prefill route's threshold (20 rows per KV head), pages of one tile
    ("g4_d64_few_queries_p64", Workload("ppf", 3, 5, 1900, 8, 2, 64, "bf16", k_global=200,
                                        window=16, needles=3, seed=708), 64),
]


@pytest.mark.parametrize("name,wl,P", CASES, ids=[c[0] for c in CASES])
def test_paged_prefill_pipeline(name, wl, P):
    say(f"[paged prefill] {name} {wl} page {P}")
    x = make_inputs(wl, device="cuda", n_sparse=1)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    kp, table = paged(k, P, wl.seed)
    vp, _ = paged(v, P, wl.seed)
    pages = (table, wl.kv_len)

    # full attention: the tiled kernel over pages, bit-identical to the contiguous call
    o, lse = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
    o2, lse2 = hs().full_attn_fwd_paged(q, kp, vp, table, wl.kv_len, out_dtype=torch.float32)
    # token and block selection from the paged K, bit-identical to the contiguous calls
    ti, tc = hs().oracle_topk(q, k, lse, wl.k_global, wl.window)
    ti2, tc2 = hs().oracle_topk(q, kp, lse2, wl.k_global, wl.window, pages=pages)
    bi, bc = hs().block_score_topk(q, k, lse, wl.block, wl.n_blocks)
    bi2, bc2 = hs().block_score_topk(q, kp, lse2, wl.block, wl.n_blocks, pages=pages)
    # the sparse layer over the paged cache and the paged token sets
    so, _ = hs().sparse_attn_gather(qs, kp, vp, ti2, tc2, kind="token", out_dtype=torch.float32,
                                    pages=pages)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(ti, ti2) and torch.equal(tc, tc2)
    assert torch.equal(bi, bi2) and torch.equal(bc, bc2)

    # against the oracle on the logical cache
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.full_attention(qn, kn, vn)
    eo = max_abs(o2.cpu().numpy(), o_ref)
    el = max_abs(lse2.cpu().numpy(), lse_ref)
    say(f"  full attention: max|dO| = {eo:.3e}, max|dLSE| = {el:.3e}")
    assert eo <= TOL_BF16 and el <= lse_bound(lse_ref)
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window)
    gi, gc = ti2.cpu().numpy(), tc2.cpu().numpy()
    ex = check_token_sets(gi, gc, oi, oc, qn, kn, lse_ref, wl.k_global, wl.window, wl.q_offset)
    obi, obc = oracle.block_topk(qn, kn, lse_ref, wl.block, wl.n_blocks)
    exb = check_block_sets(bi2.cpu().numpy(), bc2.cpu().numpy(), obi, obc, qn, kn, lse_ref,
                           wl.block, wl.q_offset)
    say(f"  near-tie differences excused: tokens {ex}, blocks {exb}")
    # sparse outputs on identical sets: the GPU's own (checked above), fed to the oracle
    so_ref, _ = oracle.masked_attention(to_numpy_f32(qs), kn, vn, gi, gc)
    es = max_abs(so.cpu().numpy(), so_ref)
    say(f"  paged token-sparse layer: max|dO| = {es:.3e}")
    assert es <= TOL_BF16


def test_paged_prefill_small_pages_take_the_row_kernel():
    """Pages smaller than a key tile: full attention runs on the row kernel, which translates
    every key; compared with the oracle (its rounding differs from the tiled kernel's)."""
    wl = Workload("pps", 1, 64, 1500, 16, 4, 128, "bf16", seed=705)
    x = make_inputs(wl, device="cuda")
    kp, table = paged(x["k"], 16, wl.seed)
    vp, _ = paged(x["v"], 16, wl.seed)
    o, lse = hs().full_attn_fwd_paged(x["q"], kp, vp, table, wl.kv_len, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.full_attention(qn, kn, vn)
    eo, el = max_abs(o.cpu().numpy(), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    say(f"[paged prefill, pages of 16] max|dO| = {eo:.3e}, max|dLSE| = {el:.3e}")
    assert eo <= TOL_BF16 and el <= lse_bound(lse_ref)


def test_paged_prefill_reads_only_its_pages():
    """Pool pages that the table does not name hold huge values; any read of them would blow up
    the outputs.  Also a table whose rows name pages in reverse order of position."""
    wl = Workload("ppr", 2, 128, 2048, 8, 2, 128, "bf16", k_global=128, window=32, seed=706)
    x = make_inputs(wl, device="cuda")
    P = 64
    mp = wl.kv_len // P
    B, T, Hkv, d = x["k"].shape
    n = B * mp + 5
    table = torch.empty((B, mp), dtype=torch.int32)
    for b in range(B):
        table[b] = torch.arange(mp - 1, -1, -1, dtype=torch.int32) + b * mp + 5
    pools = []
    for t in (x["k"], x["v"]):
        pool = torch.full((n, P, Hkv, d), 3e4, dtype=t.dtype, device="cuda")
        for b in range(B):
            for p in range(mp):
                pool[int(table[b, p])] = t[b, p * P:(p + 1) * P]
        pools.append(pool)
    table = table.cuda()
    o, lse = hs().full_attn_fwd(x["q"], x["k"], x["v"], out_dtype=torch.float32)
    o2, lse2 = hs().full_attn_fwd_paged(x["q"], pools[0], pools[1], table, wl.kv_len,
                                        out_dtype=torch.float32)
    ti, tc = hs().oracle_topk(x["q"], x["k"], lse, wl.k_global, wl.window)
    ti2, tc2 = hs().oracle_topk(x["q"], pools[0], lse2, wl.k_global, wl.window,
                                pages=(table, wl.kv_len))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(ti, ti2) and torch.equal(tc, tc2)
    assert np.isfinite(o2.cpu().numpy()).all()
