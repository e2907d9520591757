"""GPU parity of hs_full_attn_topk: full attention and the token-level oracle index in one call.
On prefill shapes the attention pass records every row's per-tile logit maximum and the
selection starts each (b, t, u), or each chunk of 16 heads of a larger group, at the k-th
largest tile score before the window (a lower bound of its k-th candidate score); elsewhere the
call is full attention followed by the separate selection.

O and LSE must equal hs_full_attn_fwd's bit for bit; index sets must equal the separate
hs_oracle_topk's exactly (the bound only decides which keys enter the candidate lists, never
which win) and the oracle's up to the near-tie rule of parity_utils.  A negative bound margin
forces bounds above the k-th score, so those rows take the second pass.
"""
import sys

import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import LSE_TOL, TOL_BF16, TOL_F32, check_token_sets, max_abs

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(x):
    return x.cuda() if torch.is_tensor(x) else x


CASES = [
    # the bound applies to the later queries: at least k whole tiles before the window
    ("g4_k16", Workload("t4", 1, 300, 3000, 8, 2, 128, "bf16", k_global=16, window=16, seed=701)),
    ("g16_k32", Workload("t16", 1, 50, 4000, 32, 2, 128, "bf16", k_global=32, window=32,
                         seed=702)),
    ("g8_d64_k24", Workload("t8", 2, 100, 3000, 16, 2, 64, "bf16", k_global=24, window=8,
                            seed=703)),
    ("g1_k20", Workload("t1", 1, 40, 2500, 4, 4, 128, "bf16", k_global=20, window=16, seed=704)),
    ("g2_k8_w0", Workload("t2", 1, 70, 1800, 8, 4, 128, "bf16", k_global=8, window=0, seed=705)),
    # causal from position 0: early queries have no bound (fewer than k tiles), later ones do
    ("g4_causal_ragged", Workload("tc", 2, 1333, 1333, 8, 2, 128, "bf16", k_global=12, window=20,
                                  seed=706)),
    # needles: a few keys far above the rest
    ("g16_needles", Workload("tn", 1, 64, 5000, 16, 1, 128, "bf16", k_global=16, window=64,
                             needles=16, seed=707)),
    # k of the 80B workload: 1024 candidates of a 70k context (1090 tiles before the window)
    ("g16_k1024", Workload("tk", 1, 32, 70000, 16, 1, 128, "bf16", k_global=1024, window=128,
                           seed=708)),
    # groups of more than 16 heads: a bound per chunk of 16 heads, chunk lists merged
    ("g32_chunks", Workload("tg", 1, 64, 4000, 64, 2, 128, "bf16", k_global=16, window=16,
                            seed=712)),
    ("mqa64_d128", Workload("tq", 1, 32, 5000, 64, 1, 128, "bf16", k_global=24, window=32,
                            seed=713)),
    # not the fused route: decode rows, fp32 inputs, a group the tiled kernel does not divide,
    # HySparse2's head shape (64 query heads on one KV head) at d 256
    ("mqa64_d256", Workload("tq2", 1, 32, 5000, 64, 1, 256, "bf16", k_global=24, window=32,
                            seed=716)),
    ("decode_g4", Workload("td", 2, 1, 5000, 32, 8, 128, "bf16", k_global=64, window=32,
                           seed=709)),
    ("f32_g4", Workload("tf", 1, 200, 1500, 8, 2, 64, "f32", k_global=16, window=16, seed=710)),
    ("g24", Workload("t24", 1, 40, 3000, 48, 2, 128, "bf16", k_global=16, window=16, seed=714)),
]


def run_case(wl, margin=1.0 / 64, oracle_rows=None):
    x = make_inputs(wl)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    o, lse, idx, cnt = hs().full_attn_topk(q, k, v, wl.k_global, wl.window,
                                            out_dtype=torch.float32, bound_margin=margin)
    torch.cuda.synchronize()
    o2, lse2 = hs().full_attn_fwd(q, k, v, out_dtype=torch.float32)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "o / lse differ from full_attn_fwd"
    i2, c2 = hs().oracle_topk(q, k, lse2, wl.k_global, wl.window)
    torch.cuda.synchronize()
    assert torch.equal(cnt, c2), "counts differ from the separate selection"
    assert torch.equal(idx, i2), "index sets differ from the separate selection"
    qn, kn = to_numpy_f32(x["q"]), to_numpy_f32(x["k"])
    o_ref, lse_ref = oracle.full_attention(qn, kn, to_numpy_f32(x["v"]), rows=oracle_rows)
    rows = list(range(wl.q_len)) if oracle_rows is None else list(oracle_rows)
    tol = TOL_F32 if wl.dtype == "f32" else TOL_BF16
    assert max_abs(o.cpu().numpy()[:, rows], o_ref[:, rows]) <= tol
    assert max_abs(lse.cpu().numpy()[:, :, rows], lse_ref[:, :, rows]) <= LSE_TOL
    return qn, kn, lse_ref, idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("name,wl", CASES, ids=[c[0] for c in CASES])
def test_full_attn_topk_matches_separate_calls_and_oracle(name, wl):
    say(f"[full_attn_topk] {name} {wl}")
    rows = None if wl.q_len * wl.kv_len <= 4_000_000 else list(range(0, wl.q_len, 7))
    qn, kn, lse_ref, gi, gc = run_case(wl, oracle_rows=rows)
    oi, oc = oracle.token_topk(qn, kn, lse_ref, wl.k_global, wl.window, rows=rows)
    excused = check_token_sets(gi, gc, oi, oc, qn, kn, lse_ref, wl.k_global, wl.window,
                               wl.q_offset, rows=rows)
    say(f"  near-tie differences excused: {excused}")


MARGIN_SHAPES = [Workload("tm", 1, 96, 4000, 16, 2, 128, "bf16", k_global=24, window=16, seed=711),
                 Workload("tm64", 1, 32, 5000, 64, 1, 128, "bf16", k_global=24, window=32,
                          seed=715)]


@pytest.mark.parametrize("margin", [-64.0, 8.0, 0.0])
@pytest.mark.parametrize("wl", MARGIN_SHAPES, ids=["g16", "mqa64_chunks"])
def test_bound_margin_never_changes_the_sets(margin, wl):
    """A bound pushed far above every k-th score (negative margin: each bounded row, or chunk
    row, collects fewer than k candidates and takes the second pass, and the chunk merge runs
    again for it), a weak one, and none: the same sets."""
    say(f"[bound margin {margin}] {wl}")
    run_case(wl, margin=margin, oracle_rows=[0, wl.q_len // 2, wl.q_len - 1])
