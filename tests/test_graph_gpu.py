"""Every stage of the decode path captured in one HIP graph (torch.cuda.CUDAGraph): replays,
interleaved with eager work and synchronizations, give exactly the eager outputs.

The library allocates nothing and never synchronizes, and all its zero-fills are kernels, so a
whole hot-path step can be captured; bench.py times the step this way.
"""
import sys

import pytest
import torch

from oracle_top_kv_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def step(wl, x):
    H = hs()
    q, k, v = x["q"], x["k"], x["v"]
    o, lse = H.full_attn_fwd(q, k, v)
    idx, cnt = H.oracle_topk(q, k, lse, wl.k_global, wl.window)
    outs = [o, lse, idx, cnt]
    for qs in x["q_sparse"]:
        outs.append(H.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")[0])
    bidx, bcnt = H.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
    og, _ = H.sparse_attn_gather(x["q_sparse"][0], k, v, bidx, bcnt, kind="block",
                                 block=wl.block, swa=(x["k_loc"], x["v_loc"], x["gate"],
                                                      wl.window))
    return outs + [bidx, bcnt, og]


def step_logits(wl, x):
    """The decode step with stored logits, the options form of the sparse layer, and the one-pass
    block selection of the prefill kernel (for prefill shapes)."""
    H = hs()
    q, k, v = x["q"], x["k"], x["v"]
    o, lse, lg = H.full_attn_fwd_logits(q, k, v)
    idx, cnt = H.oracle_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.k_global,
                                         wl.window)
    sink = x["sink"]
    # logits past a row's own position are unspecified: compare the causal part only
    outs = [o, lse, lg.masked_fill(~x["causal"], 0.0), idx, cnt]
    for qs in x["q_sparse"]:
        outs.append(H.sparse_attn_gather(qs, k, v, idx, cnt, kind="token", sink=sink,
                                          out_gate=x["out_gate"])[0])
    bidx, bcnt = H.block_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.block,
                                          wl.n_blocks)
    og, _ = H.sparse_attn_gather(x["q_sparse"][0], k, v, bidx, bcnt, kind="block",
                                 block=wl.block, swa=(x["k_loc"], x["v_loc"], x["gate"],
                                                      wl.window), sink=sink, sink_local=sink)
    outs += [bidx, bcnt, og]
    if wl.q_len > 1:
        outs += list(H.full_attn_block_topk(q, k, v, 64, wl.n_blocks))
    return outs


def check_graph(wl, x, fn):
    eager = [t.clone() for t in fn(wl, x)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn(wl, x)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static = fn(wl, x)
    for rep in range(4):
        junk = fn(wl, x)
        torch.cuda.synchronize()
        for t in static:
            t.fill_(0) if t.dtype != torch.int32 else t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(static, eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
        del junk


@pytest.mark.parametrize("wl", [
    Workload("gl_dec", 2, 1, 5000, 32, 8, 128, "bf16", n_sparse=2, needles=4, seed=83),
    Workload("gl_pf", 1, 64, 1500, 16, 4, 128, "bf16", n_sparse=1, k_global=256, window=32,
             block=64, n_blocks=4, seed=84),
], ids=["decode", "prefill"])
def test_graph_replays_match_eager_stored_logits_and_options(wl):
    say(f"[graph, stored logits and options] {wl}")
    x = make_inputs(wl, device="cuda", block_variant=True)
    g = torch.Generator().manual_seed(wl.seed)
    x["sink"] = torch.randn(wl.n_q_heads, generator=g).cuda()
    x["out_gate"] = torch.randn(wl.batch, wl.q_len, wl.n_q_heads, generator=g).cuda()
    t = wl.q_offset + torch.arange(wl.q_len, device="cuda")
    x["causal"] = (torch.arange(wl.kv_len, device="cuda")[None, :] <= t[:, None])[None, :, None, :]
    check_graph(wl, x, step_logits)
    say("  4 replays identical to the eager outputs")


@pytest.mark.parametrize("wl", [
    Workload("gr_dec", 2, 1, 5000, 32, 8, 128, "bf16", n_sparse=2, needles=4, seed=81),
    Workload("gr_pf", 1, 64, 1500, 16, 4, 128, "bf16", n_sparse=1, k_global=256, window=32,
             block=64, n_blocks=4, seed=82),
], ids=["decode", "prefill"])
def test_graph_replays_match_eager(wl):
    say(f"[graph] {wl}")
    x = make_inputs(wl, device="cuda", block_variant=True)
    eager = [t.clone() for t in step(wl, x)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            step(wl, x)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static = step(wl, x)
    for rep in range(4):
        # eager work of the program itself between the replays
        junk = step(wl, x)
        torch.cuda.synchronize()
        for t in static:
            t.fill_(0) if t.dtype != torch.int32 else t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(static, eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
        del junk
    say("  4 replays identical to the eager outputs")
