"""Pins of the CPU oracle to facts other than itself (no GPU).

Each test fixes the oracle against a library routine (torch SDPA / softmax / logsumexp in float64,
numpy sorting), a closed form, an invariant the pages state, a brute-force counting definition, or
a worked number printed on the pages (tests/golden).  Together they are chosen so that a plausible
slip anywhere in the oracle (scale, head mapping, causal bound, window bound, tie rule, group max,
block boundary, gate order) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd import costs
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, dtype=torch.float32)).numpy()


def sdpa_ref(q, k, v, q_offset, mask_fn=None, scale=None):
    """torch SDPA in float64 with GQA expanded by repeat_interleave and an explicit mask
    (scale: SDPA's own scale argument; None is its default 1/sqrt(d)).
    Returns o [B,Tq,Hq,d] and lse [B,Hq,Tq] (lse from torch.logsumexp of the masked logits)."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    qt = torch.from_numpy(q).double().permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).double().permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).double().permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    tpos = torch.arange(Tq)[:, None] + q_offset
    ipos = torch.arange(Tk)[None, :]
    mask = ipos <= tpos
    if mask_fn is not None:
        mask = mask_fn(mask)  # [..., Tq, Tk] boolean, broadcastable to [B,Hq,Tq,Tk]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * (1.0 / math.sqrt(d) if scale is None else scale)
    logits = logits.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


def softmax_probs(q, k, q_offset):
    """p[b, h, j, i] via torch.softmax (float64) of the causal logits; -inf -> 0 outside."""
    B, Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    qt = torch.from_numpy(q).double().permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).double().permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    logits = (qt @ kt.transpose(-1, -2)) / math.sqrt(d)
    mask = torch.arange(Tk)[None, :] <= (torch.arange(Tq)[:, None] + q_offset)
    return torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1).numpy()


# ------------------------------------------------------------------------------------------
# full attention: O and LSE
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,Tq,Tk,Hq,Hkv,d", [(2, 40, 40, 4, 2, 16), (1, 7, 50, 6, 3, 8),
                                             (1, 1, 33, 4, 1, 32)])
def test_full_attention_matches_torch_sdpa(B, Tq, Tk, Hq, Hkv, d):
    q, k, v = rnd((B, Tq, Hq, d), 1), rnd((B, Tk, Hkv, d), 2), rnd((B, Tk, Hkv, d), 3)
    o, lse = oracle.full_attention(q, k, v)
    o_ref, lse_ref = sdpa_ref(q, k, v, Tk - Tq)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


@pytest.mark.parametrize("scale", [0.05, 0.4])
def test_explicit_scale_matches_torch_sdpa(scale):
    """A logit scale other than 1/sqrt(d) (the descriptor's scale) against SDPA's own scale
    argument; the token and block rankings follow the same logits."""
    q, k, v = rnd((2, 9, 4, 16), 61), rnd((2, 30, 2, 16), 62), rnd((2, 30, 2, 16), 63)
    o, lse = oracle.full_attention(q, k, v, scale=scale)
    o_ref, lse_ref = sdpa_ref(q, k, v, 21, scale=scale)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12
    a = oracle.logit_row(q, k, 1, 8, 3, scale=scale)
    ref = q[1, 8, 3].astype(np.float64) @ k[1, :30, 1].astype(np.float64).T * scale
    assert np.max(np.abs(a - ref)) < 1e-12


def test_full_attention_row_subset_leaves_others():
    q, k, v = rnd((1, 20, 2, 8), 4), rnd((1, 20, 1, 8), 5), rnd((1, 20, 1, 8), 6)
    o_all, lse_all = oracle.full_attention(q, k, v)
    o, lse = oracle.full_attention(q, k, v, rows=[0, 7, 19])
    assert np.array_equal(o[:, [0, 7, 19]], o_all[:, [0, 7, 19]])
    assert np.isnan(o[:, 1]).all() and np.isnan(lse[:, :, 1]).all()


def test_identical_keys_give_prefix_mean():
    """All keys equal -> p = 1/(t+1): O = mean of V[0..t], LSE = a + ln(t+1)."""
    B, T, Hq, Hkv, d = 1, 24, 2, 1, 8
    q = rnd((B, T, Hq, d), 7)
    krow = rnd((d,), 8)
    k = np.broadcast_to(krow, (B, T, Hkv, d)).copy()
    v = rnd((B, T, Hkv, d), 9)
    o, lse = oracle.full_attention(q, k, v)
    for t in range(T):
        mean = v[0, :t + 1, 0].astype(np.float64).mean(axis=0)
        for h in range(Hq):
            a = float(np.dot(q[0, t, h].astype(np.float64), krow.astype(np.float64))) / math.sqrt(d)
            assert np.max(np.abs(o[0, t, h] - mean)) < 1e-12
            assert abs(lse[0, h, t] - (a + math.log(t + 1))) < 1e-12


def test_first_position_reads_first_value():
    q, k, v = rnd((1, 5, 2, 4), 10), rnd((1, 5, 1, 4), 11), rnd((1, 5, 1, 4), 12)
    o, _ = oracle.full_attention(q, k, v)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0].astype(np.float64))
    assert np.array_equal(o[0, 0, 1], v[0, 0, 0].astype(np.float64))


def test_logit_row_closed_form():
    """q = c e_0 per head, k_i of KV head u = (i + 10 u) e_0: a_{t,i} = c (i + 10 u) / sqrt(d) for
    i = 0..t, with u = h // g (a wrong head mapping, scale or causal length fails)."""
    B, Tq, Tk, Hq, Hkv, d = 1, 3, 9, 4, 2, 16
    q = np.zeros((B, Tq, Hq, d), np.float32)
    k = np.zeros((B, Tk, Hkv, d), np.float32)
    for h in range(Hq):
        q[0, :, h, 0] = h + 1
    for u in range(Hkv):
        k[0, :, u, 0] = np.arange(Tk) + 10 * u
    for j in range(Tq):
        t = Tk - Tq + j
        for h in range(Hq):
            a = oracle.logit_row(q, k, 0, j, h)
            assert a.shape == (t + 1,)
            want = (h + 1) * (np.arange(t + 1) + 10 * (h // 2)) / math.sqrt(d)
            assert np.max(np.abs(a - want)) < 1e-12


def test_one_hot_values_read_back_probabilities():
    """V = identity rows: O[t, h, c] = p_{t,c}; and sum_i p_{t,i} = 1."""
    T, d = 16, 16
    q, k = rnd((1, T, 2, d), 13), rnd((1, T, 1, d), 14)
    v = np.eye(T, d, dtype=np.float32)[None, :, None, :]
    o, lse = oracle.full_attention(q, k, v)
    for t in [0, 5, 15]:
        for h in range(2):
            p = oracle.prob_row(q, k, 0, t, h)
            assert abs(p.sum() - 1.0) < 1e-14
            assert np.max(np.abs(o[0, t, h, :t + 1] - p)) < 1e-14
            p2 = oracle.prob_row(q, k, 0, t, h, lse=lse)
            assert np.max(np.abs(p2 - p)) < 1e-14


# ------------------------------------------------------------------------------------------
# token scores and token top-k
# ------------------------------------------------------------------------------------------

def brute_topk_sets(score, t, k_global, window):
    """Counting definition (no sort): candidate i (i <= t-w) is selected iff fewer than k
    candidates beat it, where j beats i if s_j > s_i, or s_j == s_i and j < i."""
    nc = max(0, t - window + 1)
    s = score[:nc]
    beats = (s[None, :] > s[:, None]) | ((s[None, :] == s[:, None]) &
                                        (np.arange(nc)[None, :] < np.arange(nc)[:, None]))
    chosen = set(np.nonzero(beats.sum(axis=1) < k_global)[0].tolist())
    chosen |= set(range(max(0, t - window + 1), t + 1))
    return sorted(chosen)


def check_set_invariants(idx, cnt, k_global, window, q_offset):
    B, Tq, Hkv, cap = idx.shape
    for b in range(B):
        for j in range(Tq):
            t = q_offset + j
            for u in range(Hkv):
                n = cnt[b, j, u]
                row = idx[b, j, u]
                assert n == min(t + 1, k_global + window)
                assert (row[n:] == -1).all()
                s = row[:n]
                assert (np.diff(s) > 0).all() and s[0] >= 0 and s[-1] <= t
                win = np.arange(max(0, t - window + 1), t + 1)
                assert np.isin(win, s).all()
                if t + 1 <= k_global + window:
                    assert np.array_equal(s, np.arange(t + 1))


def test_token_topk_matches_counting_definition_and_softmax_scores():
    """Scores from torch.softmax (float64) with the group max taken in numpy, selection by the
    counting definition; tiny fp32 workload, all rows.  Includes exact ties (duplicated keys)."""
    wl = Workload("t", 1, 160, 160, 4, 2, 16, "f32", k_global=20, window=6, seed=77)
    x = make_inputs(wl)
    q, k = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    k[0, 50:60] = k[0, 10:20]  # exact score ties within each head
    k[0, 90] = k[0, 30]
    idx, cnt = oracle.token_topk(q, k, None, wl.k_global, wl.window)
    check_set_invariants(idx, cnt, wl.k_global, wl.window, 0)
    p = softmax_probs(q, k, 0)  # [B, Hq, Tq, Tk]
    g = wl.group
    for j in range(wl.q_len):
        for u in range(wl.n_kv_heads):
            s = p[0, u * g:(u + 1) * g, j, :j + 1].max(axis=0)
            want = brute_topk_sets(s, j, wl.k_global, wl.window)
            assert idx[0, j, u, :cnt[0, j, u]].tolist() == want, (j, u)


def test_token_scores_are_group_max_of_softmax():
    wl = Workload("t", 2, 6, 70, 8, 2, 16, "f32", seed=5)
    x = make_inputs(wl)
    q, k = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    _, lse = oracle.full_attention(q, k, to_numpy_f32(x["v"]))
    p = softmax_probs(q, k, wl.q_offset)
    for b in range(2):
        for j in [0, 5]:
            for u in range(2):
                s = oracle.token_score_row(q, k, lse, b, j, u)
                ref = p[b, u * 4:(u + 1) * 4, j, :wl.q_offset + j + 1].max(axis=0)
                assert np.max(np.abs(s - ref)) < 1e-15


def test_rank_invariance_single_head_group():
    """g = 1: ranking by p equals ranking by the raw logit q.k (numpy argsort, ties by
    position) [P2 'Why normalize scores for TopK']."""
    T, d, kg = 300, 32, 40
    q, k = rnd((1, T, 1, d), 21), rnd((1, T, 1, d), 22)
    idx, cnt = oracle.token_topk(q, k, None, kg, 0, cap=kg)
    for t in [39, 40, 41, 150, 299]:
        logit = k[0, :t + 1, 0].astype(np.float64) @ q[0, t, 0].astype(np.float64)
        order = np.lexsort((np.arange(t + 1), -logit))
        want = np.sort(order[:kg])
        assert np.array_equal(idx[0, t, 0, :cnt[0, t, 0]], want)


def test_identical_heads_equal_single_head():
    T, d = 120, 16
    q1, k = rnd((1, T, 1, d), 31), rnd((1, T, 1, d), 32)
    q4 = np.repeat(q1, 4, axis=2)
    a, ca = oracle.token_topk(q1, k, None, 10, 4)
    b, cb = oracle.token_topk(q4, k, None, 10, 4)
    assert np.array_equal(a, b) and np.array_equal(ca, cb)


def test_needles_are_selected():
    wl = Workload("n", 2, 1, 3000, 8, 2, 64, "f32", k_global=64, window=32, needles=6,
                  needle_logit=8.0, seed=9)
    x = make_inputs(wl)
    q, k = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    idx, cnt = oracle.token_topk(q, k, None, wl.k_global, wl.window)
    check_set_invariants(idx, cnt, wl.k_global, wl.window, wl.q_offset)
    for b in range(2):
        for u in range(2):
            sel = set(idx[b, 0, u, :cnt[b, 0, u]].tolist())
            assert set(x["needle_pos"][b, u].tolist()) <= sel
            assert all(p < wl.kv_len - wl.window for p in x["needle_pos"][b, u].tolist())


# ------------------------------------------------------------------------------------------
# sparse layer over an index set
# ------------------------------------------------------------------------------------------

def test_masked_attention_matches_sdpa_with_boolean_mask():
    wl = Workload("m", 2, 30, 90, 4, 2, 16, "f32", k_global=12, window=5, seed=41)
    x = make_inputs(wl)
    q, k, v = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    qs = to_numpy_f32(x["q_sparse"][0])
    idx, cnt = oracle.token_topk(q, k, None, wl.k_global, wl.window)
    o, lse = oracle.masked_attention(qs, k, v, idx, cnt)
    member = np.zeros((wl.batch, wl.n_kv_heads, wl.q_len, wl.kv_len), dtype=bool)
    for b in range(wl.batch):
        for j in range(wl.q_len):
            for u in range(wl.n_kv_heads):
                member[b, u, j, idx[b, j, u, :cnt[b, j, u]]] = True
    mem = torch.from_numpy(member).repeat_interleave(wl.group, dim=1)
    o_ref, lse_ref = sdpa_ref(qs, k, v, wl.q_offset, mask_fn=lambda m: m & mem)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


def test_sparse_equals_full_when_budget_covers_prefix():
    """k + w >= t + 1 for every row: the index set is the whole prefix, so the sparse layer is
    full attention with the same Q'."""
    wl = Workload("c", 1, 64, 64, 4, 1, 32, "f32", k_global=48, window=16, seed=42)
    x = make_inputs(wl)
    q, k, v = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    qs = to_numpy_f32(x["q_sparse"][0])
    idx, cnt = oracle.token_topk(q, k, None, wl.k_global, wl.window)
    o_s, lse_s = oracle.masked_attention(qs, k, v, idx, cnt)
    o_f, lse_f = oracle.full_attention(qs, k, v)
    assert np.max(np.abs(o_s - o_f)) < 1e-13 and np.max(np.abs(lse_s - lse_f)) < 1e-13


def test_retained_mass_decomposition_and_bound():
    """o_full = alpha o_S + (1 - alpha) o_Sbar exactly, and |o_full - o_S| <= 2 (1-alpha) V_max
    [P2 'Understanding the error through retained attention mass']."""
    wl = Workload("e", 1, 20, 200, 2, 1, 16, "f32", k_global=16, window=4, seed=43)
    x = make_inputs(wl)
    q, k, v = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    qs = to_numpy_f32(x["q_sparse"][0])
    idx, cnt = oracle.token_topk(q, k, None, wl.k_global, wl.window)
    o_s, _ = oracle.masked_attention(qs, k, v, idx, cnt)
    o_f, lse_f = oracle.full_attention(qs, k, v)
    comp = np.full((1, wl.q_len, 1, wl.kv_len), -1, dtype=np.int32)
    ccnt = np.zeros((1, wl.q_len, 1), dtype=np.int32)
    for j in range(wl.q_len):
        t = wl.q_offset + j
        rest = np.setdiff1d(np.arange(t + 1), idx[0, j, 0, :cnt[0, j, 0]])
        comp[0, j, 0, :len(rest)] = rest
        ccnt[0, j, 0] = len(rest)
    o_c, _ = oracle.masked_attention(qs, k, v, comp, ccnt)
    vmax = np.linalg.norm(v[0, :, 0].astype(np.float64), axis=1).max()
    for j in range(wl.q_len):
        for h in range(2):
            p = oracle.prob_row(qs, k, 0, j, h)
            alpha = p[idx[0, j, 0, :cnt[0, j, 0]]].sum()
            mix = alpha * o_s[0, j, h] + (1 - alpha) * o_c[0, j, h]
            assert np.max(np.abs(mix - o_f[0, j, h])) < 1e-13
            assert np.linalg.norm(o_f[0, j, h] - o_s[0, j, h]) <= 2 * (1 - alpha) * vmax + 1e-12


def test_masked_attention_rejects_out_of_range_index():
    q, k, v = rnd((1, 2, 1, 4), 1), rnd((1, 8, 1, 4), 2), rnd((1, 8, 1, 4), 3)
    idx = np.array([[[[0, 7]], [[0, 1]]]], dtype=np.int32)  # t = 6 for row 0: 7 is in the future
    cnt = np.array([[[2], [2]]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.masked_attention(q, k, v, idx, cnt)


# ------------------------------------------------------------------------------------------
# block scores, block top-k, gated block-sparse + SWA
# ------------------------------------------------------------------------------------------

def test_block_scores_match_algorithm1_route():
    """Store the per-block rowmax of the logits m~, then exp(m~ - m)/l with the row's global max
    m and l = sum exp(a - m) (Algorithm 1 of the HySparse paper, with the exponential its normalization step omits,
    as the part-1 notes point out).  The literal form (m~ - m)/l is negative and cannot match."""
    T, d, Bk = 200, 16, 16
    q, k = rnd((1, T, 3, d), 51), rnd((1, T, 1, d), 52)
    for t in [0, 15, 16, 63, 150, 199]:
        for h in range(3):
            a = (k[0, :t + 1, 0].astype(np.float64) @ q[0, t, h].astype(np.float64)) / math.sqrt(d)
            m = a.max()
            ell = np.exp(a - m).sum()
            nb = t // Bk + 1
            mt = np.array([a[r * Bk:min((r + 1) * Bk, t + 1)].max() for r in range(nb)])
            alg1 = np.exp(mt - m) / ell
            literal = (mt - m) / ell
            q1 = q[:, :, h:h + 1]
            got = oracle.block_score_row(q1, k, None, 0, t, 0, Bk, q_offset=0)
            assert np.max(np.abs(got - alg1)) < 1e-15
            if nb > 1:
                assert np.max(np.abs(got - literal)) > 1e-6
    # group max over heads
    got = oracle.block_score_row(q, k, None, 0, 150, 0, Bk, q_offset=0)
    per = [oracle.block_score_row(q[:, :, h:h + 1], k, None, 0, 150, 0, Bk, q_offset=0)
           for h in range(3)]
    assert np.array_equal(got, np.max(per, axis=0))


def test_block_size_one_equals_token_topk():
    """B = 1, n_blocks = k, w = 0: block selection is token selection."""
    T, d, kg = 150, 16, 24
    q, k = rnd((1, T, 4, d), 61), rnd((1, T, 2, d), 62)
    bi, bc = oracle.block_topk(q, k, None, 1, kg)
    ti, tc = oracle.token_topk(q, k, None, kg, 0, cap=kg)
    assert np.array_equal(bi, ti) and np.array_equal(bc, tc)


def test_block_topk_counting_definition():
    wl = Workload("b", 1, 64, 640, 4, 1, 16, "f32", seed=63)
    x = make_inputs(wl)
    q, k = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    Bk, nb = 32, 5
    bi, bc = oracle.block_topk(q, k, None, Bk, nb)
    for j in [0, 10, 63]:
        t = wl.q_offset + j
        s = oracle.block_score_row(q, k, None, 0, j, 0, Bk)
        n = t // Bk + 1
        beats = (s[None, :] > s[:, None]) | ((s[None, :] == s[:, None]) &
                                            (np.arange(n)[None, :] < np.arange(n)[:, None]))
        want = np.nonzero(beats.sum(axis=1) < nb)[0]
        assert bc[0, j, 0] == min(nb, n)
        assert np.array_equal(bi[0, j, 0, :bc[0, j, 0]], want)


def _gated_setup(seed, T=96, Tq=12, Hq=4, Hkv=2, d=16, Bk=16, nb=3, w=8):
    wl = Workload("g", 1, Tq, T, Hq, Hkv, d, "f32", block=Bk, n_blocks=nb, window=w, seed=seed)
    x = make_inputs(wl, block_variant=True)
    arr = {n: to_numpy_f32(x[n]) for n in ("q", "k", "v", "k_loc", "v_loc", "gate")}
    arr["qs"] = to_numpy_f32(x["q_sparse"][0])
    bi, bc = oracle.block_topk(arr["q"], arr["k"], None, Bk, nb)
    return wl, arr, bi, bc


def test_gated_branches_match_sdpa_masks():
    wl, a, bi, bc = _gated_setup(71)
    o, og, ol = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                       a["v_loc"], wl.window, a["gate"])
    member = np.zeros((1, wl.n_kv_heads, wl.q_len, wl.kv_len), dtype=bool)
    for j in range(wl.q_len):
        for u in range(wl.n_kv_heads):
            for r in bi[0, j, u, :bc[0, j, u]]:
                member[0, u, j, r * wl.block:(r + 1) * wl.block] = True
    mem = torch.from_numpy(member).repeat_interleave(wl.group, dim=1)
    og_ref, _ = sdpa_ref(a["qs"], a["k"], a["v"], wl.q_offset, mask_fn=lambda m: m & mem)
    tpos = torch.arange(wl.q_len)[:, None] + wl.q_offset
    win = torch.arange(wl.kv_len)[None, :] > tpos - wl.window
    ol_ref, _ = sdpa_ref(a["qs"], a["k_loc"], a["v_loc"], wl.q_offset, mask_fn=lambda m: m & win)
    assert np.max(np.abs(og - og_ref)) < 1e-12
    assert np.max(np.abs(ol - ol_ref)) < 1e-12
    sg = 1 / (1 + np.exp(-a["gate"][..., 0:1].astype(np.float64)))
    sl = 1 / (1 + np.exp(-a["gate"][..., 1:2].astype(np.float64)))
    assert np.max(np.abs(o - (sg * og_ref + sl * ol_ref))) < 1e-12


def test_gate_special_cases():
    wl, a, bi, bc = _gated_setup(72)
    zero = np.zeros_like(a["gate"])
    o, og, ol = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                       a["v_loc"], wl.window, zero)
    assert np.max(np.abs(o - 0.5 * (og + ol))) < 1e-14
    gl = a["gate"].copy()
    gl[..., 1] = -100.0
    o2, og2, _ = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                        a["v_loc"], wl.window, gl)
    sg = 1 / (1 + np.exp(-gl[..., 0:1].astype(np.float64)))
    assert np.max(np.abs(o2 - sg * og2)) < 1e-15


# ------------------------------------------------------------------------------------------
# per-head sink bias and sigmoid output gate of the sparse layers
# ------------------------------------------------------------------------------------------

def _sink_setup(seed, T=40, Hq=4, Hkv=2, d=16, n_idx=12):
    q = rnd((1, 1, Hq, d), seed)
    k = rnd((1, T, Hkv, d), seed + 1)
    v = rnd((1, T, Hkv, d), seed + 2)
    r = np.random.default_rng(seed)
    idx = np.full((1, 1, Hkv, n_idx), -1, np.int32)
    for u in range(Hkv):
        idx[0, 0, u] = np.sort(r.choice(T, n_idx, replace=False))
    cnt = np.full((1, 1, Hkv), n_idx, np.int32)
    return q, k, v, idx, cnt


def test_sink_equals_an_extra_key_with_zero_value():
    """A sink logit s_h is attention to one more key whose logit is s_h and whose value is 0:
    build that key explicitly (k = s sqrt(d) q / |q|^2, one per head with g = 1, placed at
    position 0) and compare with the plain masked attention of the oracle."""
    T, H, d = 40, 3, 16
    q, k, v, idx, cnt = _sink_setup(81, T=T, Hq=H, Hkv=H, d=d)
    sink = np.array([0.7, 3.5, -2.0], np.float32)  # below, near and above the typical logits
    o_s, lse_s = oracle.masked_attention(q, k, v, idx, cnt, sink=sink)
    k2 = np.zeros((1, T + 1, H, d), np.float32)
    v2 = np.zeros((1, T + 1, H, d), np.float32)
    k2[0, 1:], v2[0, 1:] = k[0], v[0]
    for h in range(H):
        qh = q[0, 0, h].astype(np.float64)
        k2[0, 0, h] = (sink[h] * math.sqrt(d) * qh / (qh @ qh)).astype(np.float32)
    idx2 = np.concatenate([np.zeros((1, 1, H, 1), np.int32), idx + 1], axis=-1)
    o_x, lse_x = oracle.masked_attention(q, k2, v2, idx2, cnt + 1)
    assert np.max(np.abs(o_s - o_x)) < 1e-6
    assert np.max(np.abs(lse_s - lse_x)) < 1e-6
    o_n, lse_n = oracle.masked_attention(q, k, v, idx, cnt)
    assert np.max(np.abs(o_s - o_n)) > 1e-3  # the sink matters here


def test_sink_limits_and_identical_keys():
    q, k, v, idx, cnt = _sink_setup(82)
    o_n, lse_n = oracle.masked_attention(q, k, v, idx, cnt)
    o_m, lse_m = oracle.masked_attention(q, k, v, idx, cnt,
                                         sink=np.full(4, -np.inf, np.float32))
    assert np.array_equal(o_m, o_n) and np.array_equal(lse_m, lse_n)
    # identical keys: every logit is a, so o = n e^a / (e^s + n e^a) * mean(v over the set)
    k1 = np.repeat(k[:, :1], k.shape[1], axis=1)
    sink = np.array([0.3, -1.0, 2.0, 5.0], np.float32)
    o, lse = oracle.masked_attention(q, k1, v, idx, cnt, sink=sink)
    n = int(cnt[0, 0, 0])
    for h in range(4):
        u = h // 2
        a = float(q[0, 0, h].astype(np.float64) @ k1[0, 0, u].astype(np.float64)) / 4.0
        mean = v[0, idx[0, 0, u], u].astype(np.float64).mean(axis=0)
        frac = n * math.exp(a) / (math.exp(float(sink[h])) + n * math.exp(a))
        assert np.max(np.abs(o[0, 0, h] - frac * mean)) < 1e-12
        assert abs(lse[0, h, 0] - math.log(math.exp(float(sink[h])) + n * math.exp(a))) < 1e-12
    # an empty set: o = 0 and LSE = the sink
    o0, l0 = oracle.masked_attention(q, k, v, np.full_like(idx, -1), np.zeros_like(cnt),
                                     sink=sink)
    assert np.all(o0 == 0) and np.allclose(l0[0, :, 0], sink, atol=0, rtol=0)


def test_output_gate_scales_the_layer():
    q, k, v, idx, cnt = _sink_setup(83)
    g = rnd((1, 1, 4), 84, 2.0)
    sink = np.array([0.1, 0.2, 0.3, 0.4], np.float32)
    o, lse = oracle.masked_attention(q, k, v, idx, cnt, sink=sink)
    og, lseg = oracle.masked_attention(q, k, v, idx, cnt, sink=sink, out_gate=g)
    sg = 1 / (1 + np.exp(-g.astype(np.float64)))
    assert np.max(np.abs(og - sg[..., None] * o)) < 1e-15
    assert np.array_equal(lse, lseg)
    wl, a, bi, bc = _gated_setup(73)
    hq = a["qs"].shape[2]
    s1, s2 = rnd((hq,), 85), rnd((hq,), 86)
    gate_o = rnd(a["qs"].shape[:3], 87)
    o3, og3, ol3 = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                          a["v_loc"], wl.window, a["gate"], sink=s1, sink_loc=s2,
                                          out_gate=gate_o)
    z = a["gate"].astype(np.float64)
    want = (1 / (1 + np.exp(-gate_o.astype(np.float64))))[..., None] * (
        1 / (1 + np.exp(-z[..., 0:1])) * og3 + 1 / (1 + np.exp(-z[..., 1:2])) * ol3)
    assert np.max(np.abs(o3 - want)) < 1e-14
    # each branch is the masked attention of its own keys with its own sink: the block set
    # expanded to its causal positions, and the window positions
    cap = wl.n_blocks * wl.block
    tok = np.full((1, wl.q_len, wl.n_kv_heads, cap), -1, np.int32)
    tcnt = np.zeros((1, wl.q_len, wl.n_kv_heads), np.int32)
    win = np.full((1, wl.q_len, wl.n_kv_heads, wl.window), -1, np.int32)
    wcnt = np.zeros_like(tcnt)
    for j in range(wl.q_len):
        t = wl.q_offset + j
        for u in range(wl.n_kv_heads):
            pos = [i for r in sorted(bi[0, j, u, :bc[0, j, u]])
                   for i in range(r * wl.block, min((r + 1) * wl.block, t + 1))]
            tok[0, j, u, :len(pos)], tcnt[0, j, u] = pos, len(pos)
            wp = list(range(max(0, t - wl.window + 1), t + 1))
            win[0, j, u, :len(wp)], wcnt[0, j, u] = wp, len(wp)
    og_ref, _ = oracle.masked_attention(a["qs"], a["k"], a["v"], tok, tcnt, sink=s1)
    ol_ref, _ = oracle.masked_attention(a["qs"], a["k_loc"], a["v_loc"], win, wcnt, sink=s2)
    assert np.max(np.abs(og3 - og_ref)) < 1e-13 and np.max(np.abs(ol3 - ol_ref)) < 1e-13
    o_plain, og_p, ol_p = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block,
                                                 a["k_loc"], a["v_loc"], wl.window, a["gate"])
    assert np.max(np.abs(og3 - og_p)) > 1e-4 and np.max(np.abs(ol3 - ol_p)) > 1e-4


def test_per_channel_gates_select_branches_channel_by_channel():
    """Per-channel gates (P2: a gate may act per head or per channel).  Logits of +-60 make each
    sigmoid exactly 1 or below 1e-26, so every channel of the output is one branch's channel:
    o_glob where zG_c = +60, zL_c = -60 and o_loc where the signs flip, in a pattern that differs
    between channels, heads and queries.  The branches themselves are pinned to SDPA above."""
    wl, a, bi, bc = _gated_setup(74)
    B, Tq, Hq, d = a["qs"].shape
    pick = (np.arange(Tq)[:, None, None] + 3 * np.arange(Hq)[None, :, None]
            + np.arange(d)[None, None, :] * np.arange(1, d + 1)[None, None, :] // 2) % 2 == 0
    pick = pick[None]  # [1, Tq, Hq, d]: True -> global branch
    gch = np.empty((B, Tq, Hq, 2, d), np.float32)
    gch[..., 0, :] = np.where(pick, 60.0, -60.0)
    gch[..., 1, :] = np.where(pick, -60.0, 60.0)
    o, og, ol = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                       a["v_loc"], wl.window, gch)
    assert np.max(np.abs(o - np.where(pick, og, ol))) < 1e-24
    # equal channels reduce to the per-head gates bit for bit, with and without output gates
    rep = np.repeat(a["gate"][..., None], d, axis=-1)
    o1, _, _ = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                      a["v_loc"], wl.window, rep)
    o2, _, _ = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                      a["v_loc"], wl.window, a["gate"])
    assert np.array_equal(o1, o2)
    gate_o = rnd(a["qs"].shape[:3], 75)
    o3, _, _ = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                      a["v_loc"], wl.window, rep,
                                      out_gate=np.repeat(gate_o[..., None], d, axis=-1))
    o4, _, _ = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                      a["v_loc"], wl.window, a["gate"], out_gate=gate_o)
    assert np.array_equal(o3, o4)
    with pytest.raises(ValueError):
        oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                               a["v_loc"], wl.window, rep, out_gate=gate_o)


def test_per_channel_output_gate_closes_or_passes_each_channel():
    """A per-channel output gate of +-60 keeps a channel whole or zeroes it (sigmoid exactly 1,
    or below 1e-26) on both the token layer and the gated layer; the LSE is unchanged."""
    q, k, v, idx, cnt = _sink_setup(88)
    B, Tq, Hq, d = q.shape
    open_ = ((np.arange(Hq)[:, None] * 5 + np.arange(d)[None, :] * 3) % 7 < 3)[None, None]
    g = np.where(open_, 60.0, -60.0).astype(np.float32)
    sink = np.array([0.1, 0.2, 0.3, 0.4], np.float32)
    o, lse = oracle.masked_attention(q, k, v, idx, cnt, sink=sink)
    oc, lsec = oracle.masked_attention(q, k, v, idx, cnt, sink=sink, out_gate=g)
    assert np.max(np.abs(oc - np.where(open_, o, 0.0))) < 1e-24
    assert np.array_equal(lse, lsec)
    wl, a, bi, bc = _gated_setup(76)
    d2 = a["qs"].shape[-1]
    rep = np.repeat(a["gate"][..., None], d2, axis=-1)
    sh = a["qs"].shape
    open2 = ((np.arange(sh[1])[:, None, None] + np.arange(sh[2])[None, :, None] * 2
              + np.arange(d2)[None, None, :]) % 3 == 0)[None]
    g2 = np.where(open2, 60.0, -60.0).astype(np.float32)
    o5, _, _ = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                      a["v_loc"], wl.window, rep, out_gate=g2)
    o6, _, _ = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, wl.block, a["k_loc"],
                                      a["v_loc"], wl.window, a["gate"])
    assert np.max(np.abs(o5 - np.where(open2, o6, 0.0))) < 1e-24


def test_blocks_covering_prefix_and_wide_window_are_full_attention():
    """B * n_blocks >= t + 1 selects every causal block; w >= t + 1 with K' = K, V' = V makes
    the local branch full attention too."""
    wl, a, _, _ = _gated_setup(73, T=64, Tq=64, Bk=16, nb=4, w=64)
    bi, bc = oracle.block_topk(a["q"], a["k"], None, 16, 4)
    o, og, ol = oracle.gated_block_swa(a["qs"], a["k"], a["v"], bi, bc, 16, a["k"], a["v"], 64,
                                       a["gate"])
    of, _ = oracle.full_attention(a["qs"], a["k"], a["v"])
    assert np.max(np.abs(og - of)) < 1e-13 and np.max(np.abs(ol - of)) < 1e-13


# ------------------------------------------------------------------------------------------
# worked numbers printed on the pages
# ------------------------------------------------------------------------------------------

def test_cost_model_worked_examples():
    gold = json.load(open(os.path.join(GOLDEN, "cost_model_worked_examples.json")))
    one = costs.kv_bytes_full_layer(1, 32768, 4, 128, 2)
    assert one == gold["one_full_layer_kv_bytes"]["value"]
    assert 49 * one // 2**20 == gold["all_full_49_layers_mib"]["value"]
    hy = (5 * one + 44 * costs.kv_bytes_full_layer(1, 128, 4, 128, 2)) / 2**20
    assert round(hy) == gold["hysparse_80b_kv_mib"]["value"]
    assert round(49 * one / 2**20 / hy, 2) == gold["reduction_at_32k"]["value"]
    assert round(5 / 49, 3) == gold["capacity_limit_ratio"]["value"]
    # the page prints the terms as about 0.102 and 0.031 and their sum as 0.133 (exact: 0.1336)
    assert abs(5 / 49 - gold["prefill_compute_ratio"]["terms"][0]) < 1e-3
    assert abs(44 / 49 * 1152 / 32768 - gold["prefill_compute_ratio"]["terms"][1]) < 1e-3
    assert abs(costs.prefill_compute_ratio(5, 44, 32768, 1024, 128) -
               gold["prefill_compute_ratio"]["value"]) < 1e-3
    assert 49 * 32768 == gold["decode_token_kv_reads_full"]["value"]
    cap = gold["hysparse2_selection"]["k_global"] + gold["hysparse2_selection"]["k_local"]
    reads = costs.decode_token_reads(5, 44, 32768, 1024, 128)
    assert reads == gold["decode_token_kv_reads_hysparse"]["value"]
    assert 5 * 32768 + 44 * cap == reads
    assert round(reads / (49 * 32768), 3) == gold["decode_read_ratio"]["value"]
    assert round(costs.block_score_elements(32768, 64) / 1e6, 2) == 16.78
    assert 1024 // 64 == gold["blocks_per_query"]["value"]


def test_oracle_index_cap_matches_worked_budget():
    """The oracle's per-query set never exceeds k + w = 1152 (the per-query read count in the
    decode example) and reaches it once t + 1 >= 1152."""
    wl = Workload("cap", 1, 3, 1400, 2, 1, 8, "f32", seed=81)
    x = make_inputs(wl)
    q, k = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    idx, cnt = oracle.token_topk(q, k, None, 1024, 128)
    assert idx.shape[-1] == 1152 and (cnt == 1152).all()
    assert costs.index_set_size(1399, 1024, 128) == 1152 and costs.index_set_size(99, 1024, 128) == 100
