"""The C ABI library without a GPU: it loads, exports every symbol include/hysparse.h declares,
and rejects invalid calls on the host before anything is enqueued (no compute call is made)."""
import ctypes
import os
import re

import pytest
import torch

from oracle_top_kv_amd import hs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hysparse.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = hs.lib()
    names = declared_functions()
    assert set(names) == set(hs.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.hs_version().decode().startswith("hysparse")


def desc(**kw):
    base = dict(batch=1, q_len=1, kv_len=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                q_offset=-1, scale=0.0, in_dtype=hs.HS_BF16, out_dtype=hs.HS_BF16)
    base.update(kw)
    return hs.AttnDesc(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), hs.HS_ERR_UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), hs.HS_ERR_INVALID_ARG),
    (dict(q_len=0), hs.HS_ERR_INVALID_ARG),
    (dict(q_offset=1024), hs.HS_ERR_INVALID_ARG),
    (dict(q_len=4, q_offset=1021), hs.HS_ERR_INVALID_ARG),
    (dict(n_q_heads=130, n_kv_heads=2), hs.HS_ERR_UNSUPPORTED),  # g = 65
    (dict(n_q_heads=128, n_kv_heads=1), hs.HS_ERR_UNSUPPORTED),  # g = 128
    (dict(head_dim=256, in_dtype=hs.HS_F32), hs.HS_ERR_UNSUPPORTED),
    (dict(in_dtype=7), hs.HS_ERR_INVALID_ARG),
])
def test_full_attn_rejects_bad_descriptions(kw, status):
    d = desc(**kw)
    rc = hs.lib().hs_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                  None)
    assert rc == status
    assert hs.lib().hs_last_error().decode()


def test_null_pointers_rejected():
    d = desc()
    assert hs.lib().hs_full_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == \
        hs.HS_ERR_INVALID_ARG
    assert hs.lib().hs_full_attn_fwd(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                    None) == hs.HS_ERR_INVALID_ARG
    assert hs.lib().hs_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, 0,
                                    None) == hs.HS_ERR_INVALID_ARG


def test_workspace_too_small_is_reported():
    d = desc(batch=8, kv_len=32768, n_q_heads=32, n_kv_heads=8)
    need = hs.lib().hs_workspace_size(hs.HS_OP_FULL_ATTN, ctypes.byref(d), 0, 0)
    assert need > 0
    rc = hs.lib().hs_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                                  None)
    assert rc == hs.HS_ERR_WORKSPACE
    need_tk = hs.lib().hs_workspace_size(hs.HS_OP_ORACLE_TOPK, ctypes.byref(d), 1024, 128)
    rc = hs.lib().hs_oracle_topk(ctypes.byref(d), FAKE, FAKE, FAKE, 1024, 128, FAKE, FAKE, FAKE,
                                 need_tk - 1, None)
    assert rc == hs.HS_ERR_WORKSPACE


def test_decode_topk_workspace_by_row_length():
    """Decode token selection: rows of up to 131072 keys need the keys (4 bytes each) and the
    histograms only; longer rows also hold the boundary list (8 bytes per key)."""
    rows = 8 * 8
    short = desc(batch=8, kv_len=32768, n_q_heads=32, n_kv_heads=8)
    need = hs.lib().hs_workspace_size(hs.HS_OP_ORACLE_TOPK, ctypes.byref(short), 1024, 128)
    assert rows * 32768 * 4 + rows * 2049 * 4 <= need <= rows * 32768 * 4 + rows * 2049 * 4 + 4096
    edge = desc(batch=8, kv_len=131072, n_q_heads=32, n_kv_heads=8)
    need = hs.lib().hs_workspace_size(hs.HS_OP_ORACLE_TOPK, ctypes.byref(edge), 1024, 128)
    assert need < rows * 131072 * 5
    long_ = desc(batch=8, kv_len=131073, n_q_heads=32, n_kv_heads=8)
    need = hs.lib().hs_workspace_size(hs.HS_OP_ORACLE_TOPK, ctypes.byref(long_), 1024, 128)
    assert need >= rows * 131073 * 12


def test_topk_argument_checks():
    d = desc()
    L = hs.lib()
    assert L.hs_oracle_topk(ctypes.byref(d), FAKE, FAKE, FAKE, -1, 128, FAKE, FAKE, FAKE, 1 << 40,
                            None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_oracle_topk(ctypes.byref(d), FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, 1 << 40,
                            None) == hs.HS_ERR_INVALID_ARG
    # every group size up to 64 and head size 256 have a route; a workspace one byte short is
    # refused before anything is enqueued
    for kw in (dict(n_q_heads=6, n_kv_heads=2), dict(n_q_heads=48, n_kv_heads=2),
               dict(n_q_heads=64, n_kv_heads=1, head_dim=256),
               dict(q_len=64, n_q_heads=24, n_kv_heads=2),
               dict(q_len=64, n_q_heads=64, n_kv_heads=1, head_dim=256)):
        dk = desc(**kw)
        need = L.hs_workspace_size(hs.HS_OP_ORACLE_TOPK, ctypes.byref(dk), 16, 4)
        assert need > 0, kw
        assert L.hs_oracle_topk(ctypes.byref(dk), FAKE, FAKE, FAKE, 16, 4, FAKE, FAKE, FAKE,
                                need - 1, None) == hs.HS_ERR_WORKSPACE, kw
        needb = L.hs_workspace_size(hs.HS_OP_BLOCK_TOPK, ctypes.byref(dk), 64, 16)
        if needb > 0:
            assert L.hs_block_score_topk(ctypes.byref(dk), FAKE, FAKE, FAKE, 64, 16, FAKE, FAKE,
                                         FAKE, needb - 1, None) == hs.HS_ERR_WORKSPACE, kw


def test_full_attn_topk_argument_checks():
    """The one-call full attention + token selection: bad k / window / margin and NULL pointers
    are refused; prefill shapes of whole groups need the tile maxima and row flags beyond the
    separate selection's buffers; a workspace one byte short is refused before any launch."""
    L = hs.lib()
    f = L.hs_full_attn_topk
    d = desc(q_len=512, kv_len=8192)  # g = 4: the tiled prefill kernel and selection
    for kg, w, m in ((-1, 128, 0.0), (0, 0, 0.0), (16, 16, float("nan")), (16, 16, float("inf"))):
        assert f(ctypes.byref(d), FAKE, FAKE, FAKE, kg, w, m, FAKE, FAKE, FAKE, FAKE, FAKE,
                 1 << 40, None) == hs.HS_ERR_INVALID_ARG, (kg, w, m)
    assert f(ctypes.byref(d), FAKE, FAKE, None, 16, 16, 0.0, FAKE, FAKE, FAKE, FAKE, FAKE,
             1 << 40, None) == hs.HS_ERR_INVALID_ARG
    need = L.hs_workspace_size(hs.HS_OP_FULL_ATTN_TOPK, ctypes.byref(d), 1024, 128)
    sel = L.hs_workspace_size(hs.HS_OP_ORACLE_TOPK, ctypes.byref(d), 1024, 128)
    tiles = (8192 + 63) // 64
    assert need >= sel + 1 * 8 * 512 * ((tiles + 15) // 16 * 16) * 2 + 512 * 2 * 4, (need, sel)
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 1024, 128, 0.0, FAKE, FAKE, FAKE, FAKE, FAKE,
             need - 1, None) == hs.HS_ERR_WORKSPACE
    # decode rows: the two calls, whose larger workspace is the size
    dd = desc(batch=2, kv_len=5000, n_q_heads=32, n_kv_heads=8)
    need_d = L.hs_workspace_size(hs.HS_OP_FULL_ATTN_TOPK, ctypes.byref(dd), 64, 32)
    assert need_d == max(L.hs_workspace_size(hs.HS_OP_FULL_ATTN, ctypes.byref(dd), 0, 0),
                         L.hs_workspace_size(hs.HS_OP_ORACLE_TOPK, ctypes.byref(dd), 64, 32))
    assert f(ctypes.byref(dd), FAKE, FAKE, FAKE, 64, 32, 0.0, FAKE, FAKE, FAKE, FAKE, FAKE,
             need_d - 1, None) == hs.HS_ERR_WORKSPACE


def test_block_topk_argument_checks():
    L = hs.lib()
    d = desc()  # g = 4
    for block, n_blocks in ((48 + 8, 16), (64, 0), (64, 65)):
        assert L.hs_block_score_topk(ctypes.byref(d), FAKE, FAKE, FAKE, block, n_blocks, FAKE, FAKE,
                                     FAKE, 1 << 40, None) == hs.HS_ERR_UNSUPPORTED
    # head size 256 with fp32 inputs has no kernel
    d2 = desc(head_dim=256, in_dtype=hs.HS_F32)
    assert L.hs_block_score_topk(ctypes.byref(d2), FAKE, FAKE, FAKE, 64, 16, FAKE, FAKE, FAKE,
                                 1 << 40, None) == hs.HS_ERR_UNSUPPORTED
    assert L.hs_last_error().decode()


def test_sparse_argument_checks():
    d = desc()
    L = hs.lib()
    assert L.hs_sparse_attn_gather(ctypes.byref(d), FAKE, FAKE, FAKE, 5, FAKE, FAKE, 8, 64, None,
                                   FAKE, None, FAKE, 1 << 40, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_sparse_attn_gather(ctypes.byref(d), FAKE, FAKE, FAKE, hs.HS_IDX_BLOCK, FAKE, FAKE,
                                   16, 0, None, FAKE, None, FAKE, 1 << 40, None) == \
        hs.HS_ERR_INVALID_ARG
    bad = hs.SwaBranch(0x1000, 0x1000, 0x1000, 0)
    assert L.hs_sparse_attn_gather(ctypes.byref(d), FAKE, FAKE, FAKE, hs.HS_IDX_BLOCK, FAKE, FAKE,
                                   16, 64, ctypes.byref(bad), FAKE, None, FAKE, 1 << 40,
                                   None) == hs.HS_ERR_INVALID_ARG


def test_logits_entry_points_argument_checks():
    L = hs.lib()
    d = desc(batch=8, kv_len=32768, n_q_heads=32, n_kv_heads=8)
    # full attention with logits: NULL or misaligned logits, too small a workspace
    assert L.hs_full_attn_fwd_logits(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                     1 << 40, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_full_attn_fwd_logits(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                     ctypes.c_void_p(0x1002), FAKE, 1 << 40, None) == \
        hs.HS_ERR_INVALID_ARG
    need = L.hs_workspace_size(hs.HS_OP_FULL_ATTN_LOGITS, ctypes.byref(d), 0, 0)
    assert need == L.hs_workspace_size(hs.HS_OP_FULL_ATTN, ctypes.byref(d), 0, 0) > 0
    assert L.hs_full_attn_fwd_logits(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     need - 1, None) == hs.HS_ERR_WORKSPACE
    # token selection from logits: any group size is accepted; budgets are checked
    need_tk = L.hs_workspace_size(hs.HS_OP_TOPK_FROM_LOGITS, ctypes.byref(d), 1024, 128)
    assert need_tk > 0
    assert L.hs_oracle_topk_from_logits(ctypes.byref(d), FAKE, FAKE, 1024, 128, FAKE, FAKE, FAKE,
                                        need_tk - 1, None) == hs.HS_ERR_WORKSPACE
    assert L.hs_oracle_topk_from_logits(ctypes.byref(d), FAKE, FAKE, -1, 128, FAKE, FAKE, FAKE,
                                        1 << 40, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_oracle_topk_from_logits(ctypes.byref(d), None, FAKE, 16, 4, FAKE, FAKE, FAKE,
                                        1 << 40, None) == hs.HS_ERR_INVALID_ARG
    d3 = desc(n_q_heads=6, n_kv_heads=2)  # g = 3
    assert L.hs_workspace_size(hs.HS_OP_TOPK_FROM_LOGITS, ctypes.byref(d3), 16, 4) > 0
    # block selection from logits: block and n_blocks checked, any group size accepted
    for block, n_blocks in ((56, 16), (64, 0), (64, 65)):
        assert L.hs_block_topk_from_logits(ctypes.byref(d), FAKE, FAKE, block, n_blocks, FAKE,
                                           FAKE, FAKE, 1 << 40, None) == hs.HS_ERR_UNSUPPORTED
    assert L.hs_workspace_size(hs.HS_OP_BLOCK_TOPK_FROM_LOGITS, ctypes.byref(d3), 64, 16) > 0
    need_bk = L.hs_workspace_size(hs.HS_OP_BLOCK_TOPK_FROM_LOGITS, ctypes.byref(d), 64, 16)
    assert L.hs_block_topk_from_logits(ctypes.byref(d), FAKE, FAKE, 64, 16, FAKE, FAKE, FAKE,
                                       need_bk - 1, None) == hs.HS_ERR_WORKSPACE


def test_sparse_options_argument_checks():
    d = desc()
    L = hs.lib()
    opts = hs.SparseOpts(None, 0x1000, None)  # a window-branch sink without a window branch
    assert L.hs_sparse_attn_gather_ex(ctypes.byref(d), FAKE, FAKE, FAKE, hs.HS_IDX_TOKEN, FAKE,
                                      FAKE, 8, 64, None, ctypes.byref(opts), FAKE, None, FAKE,
                                      1 << 40, None) == hs.HS_ERR_INVALID_ARG
    assert "sink_local" in L.hs_last_error().decode()
    opts = hs.SparseOpts(None, None, None, 0, 2)  # gates_per_channel is 0 or 1
    assert L.hs_sparse_attn_gather_ex(ctypes.byref(d), FAKE, FAKE, FAKE, hs.HS_IDX_TOKEN, FAKE,
                                      FAKE, 8, 64, None, ctypes.byref(opts), FAKE, None, FAKE,
                                      1 << 40, None) == hs.HS_ERR_INVALID_ARG
    assert "gates_per_channel" in L.hs_last_error().decode()
    names = [f[0] for f in hs.SparseOpts._fields_]
    assert names == ["sink", "sink_local", "out_gate", "local_ring", "gates_per_channel"]
    assert hs.SparseOpts.gates_per_channel.offset == 28 and ctypes.sizeof(hs.SparseOpts) == 32


def test_gate_kinds_must_agree():
    """Per-channel and per-head gates cannot be mixed in one call (the ABI has one flag); the
    binding refuses before touching any device."""
    q = torch.zeros(1, 1, 4, 16)
    k = torch.zeros(1, 8, 2, 16)
    idx = torch.zeros(1, 1, 2, 4, dtype=torch.int32)
    cnt = torch.zeros(1, 1, 2, dtype=torch.int32)
    swa = (k, k, torch.zeros(1, 1, 4, 2, 16), 4)
    with pytest.raises(ValueError, match="per head or both per channel"):
        hs.sparse_attn_gather(q, k, k, idx, cnt, swa=swa, out_gate=torch.zeros(1, 1, 4))


def test_status_strings():
    L = hs.lib()
    for s in (0, -1, -2, -3, -4):
        assert L.hs_status_string(s).decode()


def test_large_group_workspace_sizes():
    """Groups of 64 heads on one KV head (d 256): full attention with and without logits runs the
    group kernel (one size); the paged calls run the row kernel; the sparse size covers both
    sparse paths; a workspace one byte short is refused before anything is enqueued."""
    L = hs.lib()
    d = desc(batch=8, kv_len=32768, n_q_heads=64, n_kv_heads=1, head_dim=256)
    fa = L.hs_workspace_size(hs.HS_OP_FULL_ATTN, ctypes.byref(d), 0, 0)
    assert fa > 0 and fa == L.hs_workspace_size(hs.HS_OP_FULL_ATTN_LOGITS, ctypes.byref(d), 0, 0)
    assert L.hs_workspace_size(hs.HS_OP_FULL_ATTN_PAGED, ctypes.byref(d), 64, 0) > 0
    sp = L.hs_workspace_size(hs.HS_OP_SPARSE_ATTN, ctypes.byref(d), 1152, 0)
    sp_gated = L.hs_workspace_size(hs.HS_OP_SPARSE_ATTN, ctypes.byref(d), 1024, 128)
    assert sp > 0 and sp_gated > 0
    assert L.hs_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, fa - 1,
                              None) == hs.HS_ERR_WORKSPACE
    assert L.hs_sparse_attn_gather(ctypes.byref(d), FAKE, FAKE, FAKE, hs.HS_IDX_TOKEN, FAKE, FAKE,
                                   1152, 1, None, FAKE, None, FAKE, sp - 1,
                                   None) == hs.HS_ERR_WORKSPACE
    pages = hs.KvPages(0x1000, 64, 512, 4096)
    assert L.hs_sparse_attn_gather_paged(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(pages),
                                         hs.HS_IDX_TOKEN, FAKE, FAKE, 1152, 1, None, None, FAKE,
                                         None, None, 0, None) == hs.HS_ERR_WORKSPACE
    assert "workspace" in L.hs_last_error().decode()


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: without the built library every entry point raises instead of computing."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (f"import sys; sys.path.insert(0, {root!r})\n"
            "from oracle_top_kv_amd import hs\n"
            f"hs.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
            "try:\n"
            "    hs.lib()\n"
            "    print('loaded')\n"
            "except RuntimeError as e:\n"
            "    print('raised', 'missing' in str(e))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    assert "raised True" in out.stdout, out.stdout + out.stderr


@pytest.mark.parametrize("scale", [-1.0, float("nan"), float("inf")])
def test_bad_scale_rejected(scale):
    d = desc(scale=scale)
    assert hs.lib().hs_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                     None) == hs.HS_ERR_INVALID_ARG
    assert "scale" in hs.lib().hs_last_error().decode()
    assert hs.lib().hs_workspace_size(hs.HS_OP_FULL_ATTN, ctypes.byref(d), 0, 0) == 0


def test_descriptor_layout_matches_header():
    """The binding's descriptor has the header's field order: scale follows q_offset."""
    names = [f[0] for f in hs.AttnDesc._fields_]
    assert names == ["batch", "q_len", "kv_len", "n_q_heads", "n_kv_heads", "head_dim",
                     "q_offset", "scale", "in_dtype", "out_dtype"]
    assert hs.AttnDesc.scale.offset == 32 and ctypes.sizeof(hs.AttnDesc) == 48


@pytest.mark.parametrize("q_len,ring,ok", [(1, 128, True), (1, 127, False), (4, 131, True),
                                           (4, 130, False), (600, 727, True), (600, 726, False)])
def test_ring_window_must_hold_every_position_of_the_call(q_len, ring, ok):
    """A ring of local keys holds position t in slot t % ring; the q_len rows of one call read
    window + q_len - 1 distinct positions, so a shorter ring is refused before any launch."""
    L = hs.lib()
    d = desc(q_len=q_len, kv_len=4096)
    swa = hs.SwaBranch(0x1000, 0x1000, 0x1000, 128)
    opts = hs.SparseOpts(None, None, None, ring)
    # token lists of 4096 entries always take split partials, so a valid call needs workspace
    rc = L.hs_sparse_attn_gather_ex(ctypes.byref(d), FAKE, FAKE, FAKE, hs.HS_IDX_TOKEN, FAKE,
                                    FAKE, 4096, 1, ctypes.byref(swa), ctypes.byref(opts), FAKE,
                                    None, FAKE, 0, None)
    if ok:  # passes validation and stops at the missing workspace: nothing is enqueued
        assert rc == hs.HS_ERR_WORKSPACE, (rc, L.hs_last_error().decode())
    else:
        assert rc == hs.HS_ERR_INVALID_ARG
        assert "local_ring" in L.hs_last_error().decode()


@pytest.mark.parametrize("which", ["token", "block"])
def test_paged_selection_argument_checks(which):
    """The paged selection calls take prefill shapes on pages of at least 64 positions; a
    decode shape, small pages or a missing table are refused before any launch (a valid call
    stops at the missing workspace)."""
    L = hs.lib()

    def call(d, pages, ws_bytes=0):
        pg = None if pages is None else ctypes.byref(pages)
        if which == "token":
            return L.hs_oracle_topk_paged(ctypes.byref(d), FAKE, FAKE, pg, FAKE, 1024, 128, FAKE,
                                          FAKE, FAKE if ws_bytes else None, ws_bytes, None)
        return L.hs_block_score_topk_paged(ctypes.byref(d), FAKE, FAKE, pg, FAKE, 64, 16, FAKE,
                                           FAKE, FAKE if ws_bytes else None, ws_bytes, None)

    prefill = desc(q_len=512, kv_len=8192, n_q_heads=16, n_kv_heads=4)
    good = hs.KvPages(0x1000, 64, 128, 128)
    # token candidates, and the chunk lists of a 32-head group's blocks, need a workspace (a
    # 16-head group's block selection needs none: that valid call would launch, so it is not made)
    wide = prefill if which == "token" else desc(q_len=512, kv_len=8192, n_q_heads=64,
                                                 n_kv_heads=2)
    assert call(wide, good) == hs.HS_ERR_WORKSPACE, L.hs_last_error().decode()
    assert call(prefill, None) == hs.HS_ERR_INVALID_ARG
    small = hs.KvPages(0x1000, 32, 256, 256)
    assert call(prefill, small) == hs.HS_ERR_UNSUPPORTED
    assert "page_size" in L.hs_last_error().decode()
    decode = desc(q_len=1, kv_len=8192, n_q_heads=16, n_kv_heads=4)
    assert call(decode, good) == hs.HS_ERR_UNSUPPORTED
    assert "prefill" in L.hs_last_error().decode()
    short = hs.KvPages(0x1000, 64, 100, 128)  # 100 pages of 64 < 8192 positions
    assert call(prefill, short) == hs.HS_ERR_INVALID_ARG
    npo2 = hs.KvPages(0x1000, 96, 128, 128)
    assert call(prefill, npo2) == hs.HS_ERR_INVALID_ARG


def test_paged_full_attention_workspace_by_route():
    """Paged full attention of a prefill shape without logits runs on the tiled prefill kernel
    (no workspace); with logits, or on pages smaller than a key tile, on the row kernel (split
    partials); p1 other than 0 or 1 is refused."""
    L = hs.lib()
    d = desc(q_len=4096, kv_len=135168, n_q_heads=64, n_kv_heads=4)
    assert L.hs_workspace_size(hs.HS_OP_FULL_ATTN_PAGED, ctypes.byref(d), 64, 0) == 0
    assert L.hs_workspace_size(hs.HS_OP_FULL_ATTN_PAGED, ctypes.byref(d), 64, 1) > 0
    assert L.hs_workspace_size(hs.HS_OP_FULL_ATTN_PAGED, ctypes.byref(d), 16, 0) > 0
    assert L.hs_workspace_size(hs.HS_OP_FULL_ATTN_PAGED, ctypes.byref(d), 64, 2) == 0
    assert "p1" in L.hs_last_error().decode()
    assert L.hs_workspace_size(hs.HS_OP_FULL_ATTN_PAGED, ctypes.byref(d), 48, 0) == 0
