"""GPU parity of the sparse-layer options (hs_sparse_attn_gather_ex): per-head sink logits of
the global and sliding-window branches and the sigmoid gates (per head or per channel), against
the CPU oracle, on every launch form of the sparse kernels (split + combine, one 8-wave workgroup
per set, the gated layer in one workgroup, fp32 inputs).  Index sets are the oracle's own.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle_top_kv_amd.inputs import Workload, make_inputs, to_numpy_f32
from parity_utils import LSE_TOL, TOL_BF16, TOL_F32, max_abs

pytestmark = pytest.mark.gpu


def hs():
    from oracle_top_kv_amd import hs as _hs
    return _hs


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(x):
    return x.cuda() if torch.is_tensor(x) else x


def options(wl, seed, which):
    """Sink logits spread over the range of the logits (and beyond), gate logits ~ N(0, 2)."""
    g = torch.Generator().manual_seed(seed)
    hq = wl.n_q_heads
    sink = (3.0 * torch.randn(hq, generator=g)).float() if "sink" in which else None
    sink_l = (3.0 * torch.randn(hq, generator=g)).float() if "sink_local" in which else None
    gate = (2.0 * torch.randn(wl.batch, wl.q_len, hq, generator=g)).float() \
        if "out_gate" in which else None
    return sink, sink_l, gate


def np_or_none(t):
    return None if t is None else t.numpy()


TOKEN_CASES = [
    # split key lists + combine kernel (few sets)
    ("decode_g4_split", Workload("sd", 2, 1, 6000, 32, 8, 128, "bf16", seed=501),
     ("sink", "out_gate")),
    ("decode_g4_split_sink_only", Workload("sd2", 2, 1, 3000, 32, 8, 128, "bf16", seed=502),
     ("sink",)),
    # one 8-wave workgroup per set (>= 96 sets), output gate only
    ("decode_g4_wide", Workload("sw", 16, 1, 4000, 32, 8, 128, "bf16", seed=503),
     ("sink", "out_gate")),
    ("decode_g4_wide_gate_only", Workload("sw2", 16, 1, 3000, 32, 8, 128, "bf16", seed=504),
     ("out_gate",)),
    ("prefill_g4", Workload("sp", 1, 40, 1500, 8, 2, 128, "bf16", seed=505),
     ("sink", "out_gate")),
    ("tiny_f32", Workload("st", 1, 64, 512, 4, 1, 64, "f32", k_global=64, window=16, seed=506),
     ("sink", "out_gate")),
    # other group and head sizes: 16 heads at d 64, d 256 on the row kernel, 64 heads at d 256
    # (the group kernel)
    ("decode_g16_d64", Workload("s16", 2, 1, 2500, 64, 4, 64, "bf16", k_global=300, window=32,
                                seed=507), ("sink", "out_gate")),
    ("decode_g4_d256", Workload("s256", 2, 1, 2000, 8, 2, 256, "bf16", k_global=300, window=32,
                                seed=508), ("sink", "out_gate")),
    ("mqa64_d256_two_queries", Workload("sm", 1, 2, 1500, 64, 1, 256, "bf16", k_global=200,
                                        window=32, seed=509), ("sink", "out_gate")),
    # 256 queries: unsplit lists, the group kernel normalizes and gates its rows itself
    ("mqa64_d256_unsplit", Workload("smd", 1, 256, 1500, 64, 1, 256, "bf16", k_global=200,
                                    window=32, seed=510), ("sink", "out_gate")),
]


@pytest.mark.parametrize("name,wl,which", TOKEN_CASES, ids=[c[0] for c in TOKEN_CASES])
def test_sparse_token_with_sink_and_gate(name, wl, which):
    say(f"[sparse token opts] {name} {wl} {which}")
    x = make_inputs(wl, n_sparse=1)
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    oi, oc = oracle.token_topk(qn, kn, None, wl.k_global, wl.window)
    sink, _, gate = options(wl, wl.seed, which)
    qs = x["q_sparse"][0]
    o, lse = hs().sparse_attn_gather(
        to_dev(qs), to_dev(x["k"]), to_dev(x["v"]), torch.from_numpy(oi).cuda(),
        torch.from_numpy(oc).cuda(), kind="token", out_dtype=torch.float32, want_lse=True,
        sink=None if sink is None else sink.cuda(), out_gate=None if gate is None else gate.cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.masked_attention(to_numpy_f32(qs), kn, vn, oi, oc,
                                             sink=np_or_none(sink), out_gate=np_or_none(gate))
    eo, el = max_abs(o.cpu().numpy(), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    say(f"  max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
    assert eo <= (TOL_F32 if wl.dtype == "f32" else TOL_BF16)
    assert el <= LSE_TOL


GATED_CASES = [
    # both branches split: partials merged by the two-branch combine
    ("decode_g4_split", Workload("gd", 2, 1, 5000, 32, 8, 128, "bf16", block=64, n_blocks=16,
                                 window=128, seed=511)),
    ("prefill_g4_ragged", Workload("gp", 1, 70, 900, 8, 2, 128, "bf16", block=64, n_blocks=4,
                                   window=32, seed=512)),
    # at least 2048 (query, KV head) sets: both branches in one workgroup
    ("prefill_fused_g4", Workload("gf", 1, 600, 1200, 16, 4, 128, "bf16", block=64, n_blocks=4,
                                  window=32, seed=513)),
    ("prefill_fused_f32_d64", Workload("gf32", 1, 520, 600, 16, 4, 64, "f32", block=16,
                                       n_blocks=6, window=20, seed=514)),
]


@pytest.mark.parametrize("name,wl", GATED_CASES, ids=[c[0] for c in GATED_CASES])
def test_gated_layer_with_sinks_and_gate(name, wl):
    say(f"[gated opts] {name} {wl}")
    x = make_inputs(wl, block_variant=True)
    a = {n: to_numpy_f32(x[n]) for n in ("q", "k", "v", "k_loc", "v_loc", "gate")}
    qs = x["q_sparse"][0]
    bi, bc = oracle.block_topk(a["q"], a["k"], None, wl.block, wl.n_blocks)
    sink, sink_l, gate = options(wl, wl.seed, ("sink", "sink_local", "out_gate"))
    o_ref, _, _ = oracle.gated_block_swa(to_numpy_f32(qs), a["k"], a["v"], bi, bc, wl.block,
                                         a["k_loc"], a["v_loc"], wl.window, a["gate"],
                                         sink=sink.numpy(), sink_loc=sink_l.numpy(),
                                         out_gate=gate.numpy())
    o, _ = hs().sparse_attn_gather(
        to_dev(qs), to_dev(x["k"]), to_dev(x["v"]), torch.from_numpy(bi).cuda(),
        torch.from_numpy(bc).cuda(), kind="block", block=wl.block,
        swa=(to_dev(x["k_loc"]), to_dev(x["v_loc"]), to_dev(x["gate"]), wl.window),
        out_dtype=torch.float32, sink=sink.cuda(), sink_local=sink_l.cuda(),
        out_gate=gate.cuda())
    torch.cuda.synchronize()
    eo = max_abs(o.cpu().numpy(), o_ref)
    say(f"  max|dO| = {eo:.3e}")
    assert eo <= (TOL_F32 if wl.dtype == "f32" else TOL_BF16)


def channel_gates(wl, seed, n_branch_gates):
    """Per-channel gate logits ~ N(0, 2): branch gates [B,Tq,Hq,2,d] (when n_branch_gates) and
    the output gate [B,Tq,Hq,d]."""
    g = torch.Generator().manual_seed(seed)
    shp = (wl.batch, wl.q_len, wl.n_q_heads)
    zg = (2.0 * torch.randn(shp + (2, wl.head_dim), generator=g)).float() \
        if n_branch_gates else None
    zo = (2.0 * torch.randn(shp + (wl.head_dim,), generator=g)).float()
    return zg, zo


CHANNEL_TOKEN_CASES = [c for c in TOKEN_CASES if c[0] in (
    "decode_g4_split", "decode_g4_wide", "prefill_g4", "tiny_f32", "decode_g4_d256",
    "mqa64_d256_two_queries", "mqa64_d256_unsplit")]


@pytest.mark.parametrize("name,wl,which", CHANNEL_TOKEN_CASES,
                         ids=[c[0] for c in CHANNEL_TOKEN_CASES])
def test_sparse_token_with_per_channel_gate(name, wl, which):
    """The output gate per channel (hs_sparse_opts.gates_per_channel) with a sink, on the split +
    combine, 8-wave, fp32 and group-kernel forms."""
    say(f"[sparse token channel gate] {name} {wl}")
    x = make_inputs(wl, n_sparse=1)
    qn, kn, vn = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    oi, oc = oracle.token_topk(qn, kn, None, wl.k_global, wl.window)
    sink, _, _ = options(wl, wl.seed, ("sink",))
    _, zo = channel_gates(wl, wl.seed + 1, False)
    qs = x["q_sparse"][0]
    o, lse = hs().sparse_attn_gather(
        to_dev(qs), to_dev(x["k"]), to_dev(x["v"]), torch.from_numpy(oi).cuda(),
        torch.from_numpy(oc).cuda(), kind="token", out_dtype=torch.float32, want_lse=True,
        sink=sink.cuda(), out_gate=zo.cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.masked_attention(to_numpy_f32(qs), kn, vn, oi, oc,
                                             sink=sink.numpy(), out_gate=zo.numpy())
    eo, el = max_abs(o.cpu().numpy(), o_ref), max_abs(lse.cpu().numpy(), lse_ref)
    say(f"  max|dO| = {eo:.3e} max|dLSE| = {el:.3e}")
    assert eo <= (TOL_F32 if wl.dtype == "f32" else TOL_BF16)
    assert el <= LSE_TOL


@pytest.mark.parametrize("name,wl", GATED_CASES, ids=[c[0] for c in GATED_CASES])
@pytest.mark.parametrize("with_out_gate", [True, False], ids=["out_gate", "branch_only"])
def test_gated_layer_with_per_channel_gates(name, wl, with_out_gate):
    """Branch gates (zG_c, zL_c) and the output gate per channel, with sinks, on the two-branch
    combine and on the one-workgroup gated layer."""
    say(f"[gated channel gates] {name} {wl} out_gate={with_out_gate}")
    x = make_inputs(wl, block_variant=True)
    a = {n: to_numpy_f32(x[n]) for n in ("q", "k", "v", "k_loc", "v_loc")}
    qs = x["q_sparse"][0]
    bi, bc = oracle.block_topk(a["q"], a["k"], None, wl.block, wl.n_blocks)
    sink, sink_l, _ = options(wl, wl.seed, ("sink", "sink_local"))
    zg, zo = channel_gates(wl, wl.seed + 2, True)
    zo = zo if with_out_gate else None
    o_ref, _, _ = oracle.gated_block_swa(to_numpy_f32(qs), a["k"], a["v"], bi, bc, wl.block,
                                         a["k_loc"], a["v_loc"], wl.window, zg.numpy(),
                                         sink=sink.numpy(), sink_loc=sink_l.numpy(),
                                         out_gate=np_or_none(zo))
    o, _ = hs().sparse_attn_gather(
        to_dev(qs), to_dev(x["k"]), to_dev(x["v"]), torch.from_numpy(bi).cuda(),
        torch.from_numpy(bc).cuda(), kind="block", block=wl.block,
        swa=(to_dev(x["k_loc"]), to_dev(x["v_loc"]), zg.cuda(), wl.window),
        out_dtype=torch.float32, sink=sink.cuda(), sink_local=sink_l.cuda(),
        out_gate=None if zo is None else zo.cuda())
    torch.cuda.synchronize()
    eo = max_abs(o.cpu().numpy(), o_ref)
    say(f"  max|dO| = {eo:.3e}")
    assert eo <= (TOL_F32 if wl.dtype == "f32" else TOL_BF16)


@pytest.mark.parametrize("batch", [2, 16], ids=["split", "wide"])
def test_sink_with_empty_index_sets(batch):
    """No key at all: the output is 0 and the LSE is the sink (the sink is the only logit)."""
    wl = Workload("se", batch, 1, 3000, 32, 8, 128, "bf16", seed=521)
    x = make_inputs(wl, n_sparse=1)
    cap = wl.k_global + wl.window
    idx = torch.full((batch, 1, wl.n_kv_heads, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((batch, 1, wl.n_kv_heads), dtype=torch.int32, device="cuda")
    sink, _, _ = options(wl, 522, ("sink",))
    o, lse = hs().sparse_attn_gather(to_dev(x["q_sparse"][0]), to_dev(x["k"]), to_dev(x["v"]),
                                     idx, cnt, kind="token", out_dtype=torch.float32,
                                     want_lse=True, sink=sink.cuda())
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    want = sink.view(1, -1, 1).expand(batch, -1, 1)
    assert torch.allclose(lse.cpu(), want, rtol=0, atol=1e-6)


def test_sink_local_requires_the_window_branch():
    wl = Workload("sl", 1, 1, 500, 8, 2, 128, "bf16", seed=523)
    x = make_inputs(wl, n_sparse=1)
    idx = torch.zeros((1, 1, 2, 4), dtype=torch.int32, device="cuda")
    cnt = torch.ones((1, 1, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(hs().HsError):
        hs().sparse_attn_gather(to_dev(x["q_sparse"][0]), to_dev(x["k"]), to_dev(x["v"]), idx,
                                cnt, sink_local=torch.zeros(8, device="cuda"))
