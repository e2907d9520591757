"""Shared helpers of the parity tests: comparison rules for index sets and outputs.

Index sets (token or block): bit-exact except for entries whose oracle score lies within 1e-6
relative of the k-th selected score (a near-tie that fp32 arithmetic may resolve either way).
Outputs given identical index sets: max-abs 1e-2 for bf16 inputs, 1e-5 for fp32 inputs (the
output compared is requested in fp32).  LSE: max-abs 1e-6.
"""
import numpy as np
import torch

import oracle

BAND = 1e-6
TOL_BF16 = 1e-2
TOL_F32 = 1e-5
# LSE of the full layer (natural log, fp32) against the oracle's fp64 value: the selection
# normalizes logits with it, and its error enters the 1e-6 near-tie band directly
LSE_TOL = 1e-6


def lse_bound(lse_ref):
    """Bound on |LSE_gpu - LSE_oracle|: 1e-6 while every |LSE| stays below 16 (every workload of
    the pages' shape, where the fp32 spacing is 9.5e-7); beyond, for the stress profiles that push
    logits to 20 and more, two fp32 ulps of the largest |LSE| (3.8e-6 in [16, 32)): the fp32
    result holds at best half an ulp, and the fp32 dot product behind the largest logit (its raw
    value sqrt(d) times larger) carries about one more."""
    m = float(np.max(np.abs(np.asarray(lse_ref, dtype=np.float64)[np.isfinite(lse_ref)]),
                     initial=0.0))
    if m < 16.0:
        return LSE_TOL
    return 2.0 * float(np.spacing(np.float32(m)))


def check_token_sets(gpu_idx, gpu_cnt, orc_idx, orc_cnt, q, k, lse, k_global, window, q_offset,
                     rows=None, band=BAND):
    """Compare GPU and oracle token index sets row by row.  q, k float32 numpy; lse float64
    (the oracle's own).  Returns the number of excused near-tie differences."""
    B, Tq, Hkv, cap = orc_idx.shape
    excused = 0
    js = range(Tq) if rows is None else rows
    for b in range(B):
        for j in js:
            t = q_offset + j
            for u in range(Hkv):
                n = int(orc_cnt[b, j, u])
                assert int(gpu_cnt[b, j, u]) == n, (b, j, u, int(gpu_cnt[b, j, u]), n)
                g = gpu_idx[b, j, u]
                assert (g[n:] == -1).all(), "padding"
                gs = g[:n]
                assert (np.diff(gs) > 0).all(), "ascending and unique"
                os_ = orc_idx[b, j, u, :n]
                if np.array_equal(gs, os_):
                    continue
                diff = np.setxor1d(gs, os_)
                win0 = max(0, t - window + 1)
                assert (diff < win0).all(), "window entries differ"
                s = oracle.token_score_row(q, k, lse, b, j, u, q_offset=q_offset)
                sel = os_[os_ < win0]
                s_k = s[sel].min()
                bad = [int(i) for i in diff if abs(s[i] - s_k) > band * s_k]
                assert not bad, (f"row {(b, j, u)}: tokens {bad[:8]} differ outside the tie band; "
                                 f"gaps {[float((s[i] - s_k) / s_k) for i in bad[:8]]}")
                excused += len(diff)
    return excused


def check_block_sets(gpu_idx, gpu_cnt, orc_idx, orc_cnt, q, k, lse, block, q_offset, rows=None,
                     band=BAND):
    B, Tq, Hkv, nb = orc_idx.shape
    excused = 0
    js = range(Tq) if rows is None else rows
    for b in range(B):
        for j in js:
            for u in range(Hkv):
                n = int(orc_cnt[b, j, u])
                assert int(gpu_cnt[b, j, u]) == n, (b, j, u)
                g = gpu_idx[b, j, u]
                assert (g[n:] == -1).all()
                gs = g[:n]
                assert (np.diff(gs) > 0).all()
                os_ = orc_idx[b, j, u, :n]
                if np.array_equal(gs, os_):
                    continue
                diff = np.setxor1d(gs, os_)
                s = oracle.block_score_row(q, k, lse, b, j, u, block, q_offset=q_offset)
                s_k = s[os_].min()
                bad = [int(r) for r in diff if abs(s[r] - s_k) > band * s_k]
                assert not bad, f"row {(b, j, u)}: blocks {bad} differ outside the tie band"
                excused += len(diff)
    return excused


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def paged(t, page_size, seed, spare=3):
    """[B, T, Hkv, d] -> (pool [n_pages, P, Hkv, d], block_table [B, max_pages]): every logical
    page of every batch entry in its own physical page, in a shuffled order, with a few unused
    pages in the pool (filled with large values that must never be read)."""
    B, T, Hkv, d = t.shape
    mp = (T + page_size - 1) // page_size
    n = B * mp + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n, generator=g)[:B * mp].view(B, mp).to(torch.int32)
    pool = torch.full((n, page_size, Hkv, d), 1e4, dtype=t.dtype, device=t.device)
    for b in range(B):
        for p in range(mp):
            rows = t[b, p * page_size:(p + 1) * page_size]
            pool[perm[b, p], :rows.shape[0]] = rows
    return pool, perm.to(t.device)
