"""The C ABI library without a GPU: it loads, exports every symbol include/hysparse.h declares,
and rejects invalid calls on the host before anything is enqueued (no compute call is made)."""
import ctypes
import os
import re

import pytest

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
                q_offset=-1, in_dtype=hs.HS_BF16, out_dtype=hs.HS_BF16)
    base.update(kw)
    return hs.AttnDesc(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), hs.HS_ERR_UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), hs.HS_ERR_INVALID_ARG),
    (dict(q_len=0), hs.HS_ERR_INVALID_ARG),
    (dict(q_offset=1024), hs.HS_ERR_INVALID_ARG),
    (dict(q_len=4, q_offset=1021), hs.HS_ERR_INVALID_ARG),
    (dict(n_q_heads=40, n_kv_heads=2), hs.HS_ERR_UNSUPPORTED),   # g = 20: not a multiple of 16
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
    d3 = desc(n_q_heads=6, n_kv_heads=2)  # g = 3
    assert L.hs_oracle_topk(ctypes.byref(d3), FAKE, FAKE, FAKE, 16, 4, FAKE, FAKE, FAKE, 1 << 40,
                            None) == hs.HS_ERR_UNSUPPORTED


def test_block_topk_argument_checks():
    L = hs.lib()
    d = desc()  # g = 4
    for block, n_blocks in ((48 + 8, 16), (64, 0), (64, 65)):
        assert L.hs_block_score_topk(ctypes.byref(d), FAKE, FAKE, FAKE, block, n_blocks, FAKE, FAKE,
                                     FAKE, 1 << 40, None) == hs.HS_ERR_UNSUPPORTED
    d2 = desc(n_q_heads=4, n_kv_heads=2)  # g = 2
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
