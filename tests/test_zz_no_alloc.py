"""The no-allocation sparse-layer entry point (hs_sparse_attn_gather_noalloc) against the
workspace entry point (hs_sparse_attn_gather) it varies: same kernels, so the outputs must agree
bit for bit.  Two calls in a row share the device scratch; the second one is smaller, so stale
partials of the first would show."""
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


CASES = [
    # (name, first workload, second (smaller) workload, kind)
    ("token_decode", Workload("na1", 8, 1, 32768, 32, 8, 128, "bf16", k_global=1024, window=128,
                              seed=901),
     Workload("na2", 2, 1, 5000, 32, 8, 128, "bf16", k_global=256, window=64, seed=902), "token"),
    ("gated_decode", Workload("na3", 4, 1, 20000, 32, 8, 128, "bf16", block=64, n_blocks=16,
                              window=128, seed=903),
     Workload("na4", 1, 1, 3000, 16, 4, 128, "bf16", block=64, n_blocks=8, window=32, seed=904),
     "block"),
    ("token_short_block_f32", Workload("na5", 2, 3, 2000, 8, 2, 64, "f32", k_global=300,
                                       window=32, seed=905),
     Workload("na6", 1, 2, 900, 8, 2, 64, "f32", k_global=100, window=16, seed=906), "token"),
]


def run_pair(wl, kind):
    x = make_inputs(wl, device="cuda", block_variant=kind == "block")
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    _, lse = hs().full_attn_fwd(q, k, v)
    if kind == "token":
        idx, cnt = hs().oracle_topk(q, k, lse, wl.k_global, wl.window)
        swa = None
    else:
        idx, cnt = hs().block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        swa = (x["k_loc"], x["v_loc"], x["gate"], wl.window)
    ref, ref_lse = hs().sparse_attn_gather(qs, k, v, idx, cnt, kind=kind, block=wl.block,
                                           swa=swa, out_dtype=torch.float32, want_lse=True)
    o = torch.full(qs.shape, float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full(ref_lse.shape, float("nan"), dtype=torch.float32, device="cuda")
    hs().sparse_attn_gather_noalloc(qs, k, v, idx, cnt, o, l, kind=kind, block=wl.block,
                                    swa=swa)
    torch.cuda.synchronize()
    return ref, ref_lse, o, l


@pytest.mark.parametrize("name,wl1,wl2,kind", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_entry_point(name, wl1, wl2, kind):
    for wl in (wl1, wl2):
        say(f"[no-alloc sparse layer] {name} {wl}")
        ref, ref_lse, o, l = run_pair(wl, kind)
        assert torch.equal(ref, o), float((ref - o).abs().max())
        assert torch.equal(ref_lse, l)


def test_noalloc_rejects_layers_beyond_its_scratch():
    """A layer whose split partials exceed the 16 MiB scratch is refused before any launch."""
    L = hs().lib()
    d = hs().AttnDesc(64, 1, 2 << 20, 64, 8, 128, -1, 0.0, hs().HS_BF16, hs().HS_BF16)
    need = L.hs_workspace_size(hs().HS_OP_SPARSE_ATTN, d, 16384, 0)
    assert need > 16 << 20
    fake = hs().ctypes.c_void_p(0x1000)
    rc = L.hs_sparse_attn_gather_noalloc(d, fake, fake, fake, hs().HS_IDX_TOKEN, fake, fake,
                                         16384, 1, None, fake, None, None)
    assert rc == hs().HS_ERR_WORKSPACE
    assert "no-allocation" in L.hs_last_error().decode()
