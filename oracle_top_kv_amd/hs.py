"""Thin ctypes binding of libhysparse.so (C ABI: include/hysparse.h).

Argument marshalling only: shapes and dtypes are read off torch tensors, outputs and workspace are
allocated with torch on the tensors' device, and the call is enqueued on torch's current stream.
Every step of the computation runs in the library's HIP kernels; there is no fallback.  Loading
fails loudly when the library has not been built.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhysparse.so")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_UNSUPPORTED, HS_ERR_WORKSPACE, HS_ERR_HIP = 0, -1, -2, -3, -4
HS_BF16, HS_F32 = 0, 1
HS_IDX_TOKEN, HS_IDX_BLOCK = 0, 1
HS_OP_FULL_ATTN, HS_OP_ORACLE_TOPK, HS_OP_BLOCK_TOPK, HS_OP_SPARSE_ATTN = 0, 1, 2, 3
HS_OP_FULL_ATTN_LOGITS, HS_OP_TOPK_FROM_LOGITS, HS_OP_BLOCK_TOPK_FROM_LOGITS = 4, 5, 6
HS_OP_FULL_ATTN_BLOCK_TOPK, HS_OP_FULL_ATTN_PAGED, HS_OP_FULL_ATTN_TOPK = 7, 8, 9

EXPORTS = ["hs_full_attn_fwd", "hs_oracle_topk", "hs_block_score_topk", "hs_sparse_attn_gather",
           "hs_full_attn_fwd_logits", "hs_oracle_topk_from_logits", "hs_block_topk_from_logits",
           "hs_full_attn_block_topk", "hs_sparse_attn_gather_ex", "hs_full_attn_fwd_paged",
           "hs_sparse_attn_gather_paged", "hs_sparse_attn_gather_noalloc", "hs_full_attn_topk",
           "hs_oracle_topk_paged", "hs_block_score_topk_paged", "hs_workspace_size", "hs_status_string", "hs_last_error", "hs_version"]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_offset", ctypes.c_int64),
                ("scale", ctypes.c_float), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int)]


class SwaBranch(ctypes.Structure):
    _fields_ = [("k_local", ctypes.c_void_p), ("v_local", ctypes.c_void_p),
                ("gate_logits", ctypes.c_void_p), ("window", ctypes.c_int32)]


class SparseOpts(ctypes.Structure):
    _fields_ = [("sink", ctypes.c_void_p), ("sink_local", ctypes.c_void_p),
                ("out_gate", ctypes.c_void_p), ("local_ring", ctypes.c_int32),
                ("gates_per_channel", ctypes.c_int32)]


class KvPages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


class HsError(RuntimeError):
    def __init__(self, status, what, detail):
        super().__init__(f"{what}: status {status} ({detail})")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pd = ctypes.POINTER(AttnDesc)
        L.hs_full_attn_fwd.argtypes = [pd, vp, vp, vp, vp, vp, vp, sz, vp]
        L.hs_oracle_topk.argtypes = [pd, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.hs_block_score_topk.argtypes = [pd, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.hs_sparse_attn_gather.argtypes = [pd, vp, vp, vp, ctypes.c_int, vp, vp, i32, i32,
                                            ctypes.POINTER(SwaBranch), vp, vp, vp, sz, vp]
        L.hs_full_attn_fwd_logits.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.hs_oracle_topk_from_logits.argtypes = [pd, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.hs_block_topk_from_logits.argtypes = [pd, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.hs_full_attn_block_topk.argtypes = [pd, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz,
                                              vp]
        L.hs_full_attn_topk.argtypes = [pd, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp, vp, vp,
                                        vp, sz, vp]
        L.hs_sparse_attn_gather_ex.argtypes = [pd, vp, vp, vp, ctypes.c_int, vp, vp, i32, i32,
                                               ctypes.POINTER(SwaBranch),
                                               ctypes.POINTER(SparseOpts), vp, vp, vp, sz, vp]
        pp = ctypes.POINTER(KvPages)
        L.hs_full_attn_fwd_paged.argtypes = [pd, vp, vp, vp, pp, vp, vp, vp, vp, sz, vp]
        L.hs_oracle_topk_paged.argtypes = [pd, vp, vp, pp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.hs_block_score_topk_paged.argtypes = [pd, vp, vp, pp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.hs_sparse_attn_gather_paged.argtypes = [pd, vp, vp, vp, pp, ctypes.c_int, vp, vp, i32,
                                                  i32, ctypes.POINTER(SwaBranch),
                                                  ctypes.POINTER(SparseOpts), vp, vp, vp, sz, vp]
        L.hs_sparse_attn_gather_noalloc.argtypes = [pd, vp, vp, vp, ctypes.c_int, vp, vp, i32,
                                                    i32, ctypes.POINTER(SwaBranch), vp, vp, vp]
        L.hs_workspace_size.argtypes = [ctypes.c_int, pd, i32, i32]
        L.hs_workspace_size.restype = sz
        L.hs_status_string.restype = ctypes.c_char_p
        L.hs_status_string.argtypes = [ctypes.c_int]
        L.hs_last_error.restype = ctypes.c_char_p
        L.hs_version.restype = ctypes.c_char_p
        for f in ("hs_full_attn_fwd", "hs_oracle_topk", "hs_block_score_topk",
                  "hs_sparse_attn_gather", "hs_full_attn_fwd_logits",
                  "hs_oracle_topk_from_logits", "hs_block_topk_from_logits",
                  "hs_full_attn_block_topk", "hs_sparse_attn_gather_ex",
                  "hs_full_attn_fwd_paged", "hs_sparse_attn_gather_paged",
                  "hs_sparse_attn_gather_noalloc", "hs_full_attn_topk", "hs_oracle_topk_paged",
                  "hs_block_score_topk_paged"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status, what):
    if status != HS_OK:
        raise HsError(status, what, lib().hs_last_error().decode())


def _dtype_code(t):
    if t == torch.bfloat16:
        return HS_BF16
    if t == torch.float32:
        return HS_F32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, device, dtype=None, shape=None):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def make_desc(q, k, q_offset=None, out_dtype=None, scale=None):
    B, Tq, Hq, d = q.shape
    Bk, Tk, Hkv, dk = k.shape
    if B != Bk or d != dk:
        raise ValueError("q and k shapes disagree")
    out = q.dtype if out_dtype is None else out_dtype
    return AttnDesc(B, Tq, Tk, Hq, Hkv, d, -1 if q_offset is None else int(q_offset),
                    _scale(scale), _dtype_code(q.dtype), _dtype_code(out))


def _scale(scale):
    """The descriptor's logit scale: 0 asks for the default 1/sqrt(head_dim)."""
    return 0.0 if scale is None else float(scale)


def workspace(op, desc, p0=0, p1=0, device=None):
    n = lib().hs_workspace_size(op, ctypes.byref(desc), int(p0), int(p1))
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def full_attn_fwd(q, k, v, q_offset=None, out_dtype=None, scale=None):
    """Full causal GQA attention. Returns (o [B,Tq,Hq,d], lse fp32 [B,Hq,Tq])."""
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dev, dtype=q.dtype)
    desc = make_desc(q, k, q_offset, out_dtype, scale)
    o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=dev)
    ws, n = workspace(HS_OP_FULL_ATTN, desc, device=dev)
    _check(lib().hs_full_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(lse), _ptr(ws), n, _stream(dev)), "hs_full_attn_fwd")
    return o, lse


def _pages(k_pool, block_table, page_size, dev):
    _need(block_table, "block_table", dev, dtype=torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_pages]")
    return KvPages(block_table.data_ptr(), int(page_size), int(block_table.shape[1]),
                   int(k_pool.shape[0]))


def _paged_desc(q, k_pool, kv_len, q_offset, out_dtype, scale=None):
    B, Tq, Hq, d = q.shape
    n_pages, P, Hkv, dk = k_pool.shape
    if d != dk:
        raise ValueError("q and the page pool disagree on head_dim")
    out = q.dtype if out_dtype is None else out_dtype
    return AttnDesc(B, Tq, int(kv_len), Hq, Hkv, d, -1 if q_offset is None else int(q_offset),
                    _scale(scale), _dtype_code(q.dtype), _dtype_code(out))


def full_attn_fwd_paged(q, k_pool, v_pool, block_table, kv_len, logits=False, q_offset=None,
                        out_dtype=None, scale=None):
    """Full attention over a paged cache: k_pool, v_pool [n_pages, page_size, Hkv, d],
    block_table int32 [B, max_pages].  Returns (o, lse) or (o, lse, logits)."""
    dev = q.device
    for t, n in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _need(t, n, dev, dtype=q.dtype)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool shapes differ")
    desc = _paged_desc(q, k_pool, kv_len, q_offset, out_dtype, scale)
    pg = _pages(k_pool, block_table, k_pool.shape[1], dev)
    o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=dev)
    lg = (torch.empty((q.shape[0], q.shape[1], q.shape[2], int(kv_len)), dtype=torch.float32,
                      device=dev) if logits else None)
    ws, n = workspace(HS_OP_FULL_ATTN_PAGED, desc, k_pool.shape[1], 1 if logits else 0,
                      device=dev)
    _check(lib().hs_full_attn_fwd_paged(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        ctypes.byref(pg), _ptr(o), _ptr(lse), _ptr(lg), _ptr(ws),
                                        n, _stream(dev)), "hs_full_attn_fwd_paged")
    return (o, lse, lg) if logits else (o, lse)


def full_attn_block_topk(q, k, v, block, n_blocks, q_offset=None, out_dtype=None, scale=None):
    """Full attention and the top n_blocks causal blocks in one call (one pass for prefill).
    Returns (o, lse, blk_idx int32 [B,Tq,Hkv,n_blocks], count)."""
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dev, dtype=q.dtype)
    desc = make_desc(q, k, q_offset, out_dtype, scale)
    B, Tq, Hq = q.shape[0], q.shape[1], q.shape[2]
    Hkv = k.shape[2]
    o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Tq, Hkv, n_blocks), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Tq, Hkv), dtype=torch.int32, device=dev)
    ws, n = workspace(HS_OP_FULL_ATTN_BLOCK_TOPK, desc, block, n_blocks, device=dev)
    _check(lib().hs_full_attn_block_topk(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                         int(block), int(n_blocks), _ptr(o), _ptr(lse), _ptr(idx),
                                         _ptr(cnt), _ptr(ws), n, _stream(dev)),
           "hs_full_attn_block_topk")
    return o, lse, idx, cnt


def full_attn_topk(q, k, v, k_global, window, q_offset=None, out_dtype=None, scale=None,
                   bound_margin=1.0 / 64):
    """Full attention and the forced window plus top-k_global tokens in one call (prefill: the
    selection starts at the tile-maximum bound).  Returns (o, lse, idx int32 [B,Tq,Hkv,k+w],
    count), equal to full_attn_fwd followed by oracle_topk."""
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dev, dtype=q.dtype)
    desc = make_desc(q, k, q_offset, out_dtype, scale)
    B, Tq, Hq = q.shape[0], q.shape[1], q.shape[2]
    Hkv = k.shape[2]
    o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Tq, Hkv, k_global + window), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Tq, Hkv), dtype=torch.int32, device=dev)
    ws, n = workspace(HS_OP_FULL_ATTN_TOPK, desc, k_global, window, device=dev)
    _check(lib().hs_full_attn_topk(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), int(k_global),
                                   int(window), float(bound_margin), _ptr(o), _ptr(lse),
                                   _ptr(idx), _ptr(cnt), _ptr(ws), n, _stream(dev)),
           "hs_full_attn_topk")
    return o, lse, idx, cnt


def full_attn_fwd_logits(q, k, v, q_offset=None, out_dtype=None, scale=None):
    """Full attention that also keeps its dot products q.k (decode).
    Returns (o, lse, logits fp32 [B,Tq,Hq,Tk]); logits past a row's position are unspecified."""
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dev, dtype=q.dtype)
    desc = make_desc(q, k, q_offset, out_dtype, scale)
    o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=dev)
    logits = torch.empty((q.shape[0], q.shape[1], q.shape[2], k.shape[1]), dtype=torch.float32,
                         device=dev)
    ws, n = workspace(HS_OP_FULL_ATTN_LOGITS, desc, device=dev)
    _check(lib().hs_full_attn_fwd_logits(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                         _ptr(lse), _ptr(logits), _ptr(ws), n, _stream(dev)),
           "hs_full_attn_fwd_logits")
    return o, lse, logits


def _logits_desc(logits, n_kv_heads, head_dim, q_offset, scale=None):
    B, Tq, Hq, Tk = logits.shape
    return AttnDesc(B, Tq, Tk, Hq, int(n_kv_heads), int(head_dim),
                    -1 if q_offset is None else int(q_offset), _scale(scale), HS_F32, HS_F32)


def oracle_topk_from_logits(logits, lse, n_kv_heads, head_dim, k_global, window, q_offset=None,
                            scale=None):
    """oracle_topk from the logits kept by full_attn_fwd_logits. Returns (idx, count)."""
    dev = logits.device
    _need(logits, "logits", dev, dtype=torch.float32)
    B, Tq, Hq, Tk = logits.shape
    _need(lse, "lse", dev, dtype=torch.float32, shape=(B, Hq, Tq))
    desc = _logits_desc(logits, n_kv_heads, head_dim, q_offset, scale)
    idx = torch.empty((B, Tq, n_kv_heads, k_global + window), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Tq, n_kv_heads), dtype=torch.int32, device=dev)
    ws, n = workspace(HS_OP_TOPK_FROM_LOGITS, desc, k_global, window, device=dev)
    _check(lib().hs_oracle_topk_from_logits(ctypes.byref(desc), _ptr(logits), _ptr(lse),
                                            int(k_global), int(window), _ptr(idx), _ptr(cnt),
                                            _ptr(ws), n, _stream(dev)),
           "hs_oracle_topk_from_logits")
    return idx, cnt


def block_topk_from_logits(logits, lse, n_kv_heads, head_dim, block, n_blocks, q_offset=None,
                           scale=None):
    """block_score_topk from the logits kept by full_attn_fwd_logits. Returns (blk_idx, count)."""
    dev = logits.device
    _need(logits, "logits", dev, dtype=torch.float32)
    B, Tq, Hq, Tk = logits.shape
    _need(lse, "lse", dev, dtype=torch.float32, shape=(B, Hq, Tq))
    desc = _logits_desc(logits, n_kv_heads, head_dim, q_offset, scale)
    idx = torch.empty((B, Tq, n_kv_heads, n_blocks), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Tq, n_kv_heads), dtype=torch.int32, device=dev)
    ws, n = workspace(HS_OP_BLOCK_TOPK_FROM_LOGITS, desc, block, n_blocks, device=dev)
    _check(lib().hs_block_topk_from_logits(ctypes.byref(desc), _ptr(logits), _ptr(lse),
                                           int(block), int(n_blocks), _ptr(idx), _ptr(cnt),
                                           _ptr(ws), n, _stream(dev)),
           "hs_block_topk_from_logits")
    return idx, cnt


def _select_desc(q, k, lse, q_offset, scale, pages):
    dev = q.device
    _need(q, "q", dev)
    _need(k, "k", dev, dtype=q.dtype)
    _need(lse, "lse", dev, dtype=torch.float32, shape=(q.shape[0], q.shape[2], q.shape[1]))
    if pages is None:
        return make_desc(q, k, q_offset, scale=scale), None
    desc = _paged_desc(q, k, pages[1], q_offset, q.dtype, scale)
    return desc, _pages(k, pages[0], k.shape[1], dev)


def oracle_topk(q, k, lse, k_global, window, q_offset=None, scale=None, pages=None):
    """Forced window plus top-k_global tokens. Returns (idx int32 [B,Tq,Hkv,k+w], count).
    pages = (block_table int32 [B, max_pages], kv_len): k is a page pool [n_pages, page_size,
    Hkv, d] (hs_oracle_topk_paged; prefill shapes)."""
    dev = q.device
    desc, pg = _select_desc(q, k, lse, q_offset, scale, pages)
    B, Tq, Hkv = q.shape[0], q.shape[1], k.shape[2]
    idx = torch.empty((B, Tq, Hkv, k_global + window), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Tq, Hkv), dtype=torch.int32, device=dev)
    ws, n = workspace(HS_OP_ORACLE_TOPK, desc, k_global, window, device=dev)
    if pg is None:
        _check(lib().hs_oracle_topk(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse),
                                    int(k_global), int(window), _ptr(idx), _ptr(cnt), _ptr(ws), n,
                                    _stream(dev)), "hs_oracle_topk")
    else:
        _check(lib().hs_oracle_topk_paged(ctypes.byref(desc), _ptr(q), _ptr(k), ctypes.byref(pg),
                                          _ptr(lse), int(k_global), int(window), _ptr(idx),
                                          _ptr(cnt), _ptr(ws), n, _stream(dev)),
               "hs_oracle_topk_paged")
    return idx, cnt


def block_score_topk(q, k, lse, block, n_blocks, q_offset=None, scale=None, pages=None):
    """Top n_blocks causal blocks. Returns (blk_idx int32 [B,Tq,Hkv,n_blocks], count).
    pages: as oracle_topk (hs_block_score_topk_paged)."""
    dev = q.device
    desc, pg = _select_desc(q, k, lse, q_offset, scale, pages)
    B, Tq, Hkv = q.shape[0], q.shape[1], k.shape[2]
    idx = torch.empty((B, Tq, Hkv, n_blocks), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Tq, Hkv), dtype=torch.int32, device=dev)
    ws, n = workspace(HS_OP_BLOCK_TOPK, desc, block, n_blocks, device=dev)
    if pg is None:
        _check(lib().hs_block_score_topk(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse),
                                         int(block), int(n_blocks), _ptr(idx), _ptr(cnt),
                                         _ptr(ws), n, _stream(dev)), "hs_block_score_topk")
    else:
        _check(lib().hs_block_score_topk_paged(ctypes.byref(desc), _ptr(q), _ptr(k),
                                               ctypes.byref(pg), _ptr(lse), int(block),
                                               int(n_blocks), _ptr(idx), _ptr(cnt), _ptr(ws), n,
                                               _stream(dev)), "hs_block_score_topk_paged")
    return idx, cnt


def sparse_attn_gather(q, k, v, idx, count, kind="token", block=64, swa=None, q_offset=None,
                       out_dtype=None, want_lse=False, sink=None, sink_local=None, out_gate=None,
                       local_ring=0, pages=None, scale=None):
    """Sparse layer over the shared K, V and index set with the layer's own q.
    swa = (k_local, v_local, gate_logits fp32 [B,Tq,Hq,2], window) adds the gated sliding-window
    branch; local_ring > 0: k_local / v_local are rings [B, local_ring, Hkv, d].
    sink / sink_local: fp32 [Hq] per-head sink logits of the global / window branch;
    out_gate: fp32 [B,Tq,Hq] sigmoid output-gate logits (hs_sparse_attn_gather_ex).
    Per-channel gates: gate_logits [B,Tq,Hq,2,d] and / or out_gate [B,Tq,Hq,d] (both per channel
    when both are given; sets hs_sparse_opts.gates_per_channel).
    pages = (block_table int32 [B, max_pages], kv_len): k, v are page pools
    [n_pages, page_size, Hkv, d] (hs_sparse_attn_gather_paged).  Returns (o, lse or None)."""
    per_ch = [t.dim() == q.dim() + (1 if i == 0 else 0)
              for i, t in enumerate((swa[2] if swa is not None else None, out_gate))
              if t is not None]
    if len(set(per_ch)) > 1:
        raise ValueError("gate_logits and out_gate must both be per head or both per channel")
    gate_ch = int(bool(per_ch) and per_ch[0])
    dev = q.device
    _need(q, "q", dev)
    _need(k, "k", dev, dtype=q.dtype)
    _need(v, "v", dev, dtype=q.dtype)
    _need(idx, "idx", dev, dtype=torch.int32)
    _need(count, "count", dev, dtype=torch.int32, shape=idx.shape[:3])
    if pages is not None:
        desc = _paged_desc(q, k, pages[1], q_offset, out_dtype, scale)
        pg = _pages(k, pages[0], k.shape[1], dev)
    else:
        desc = make_desc(q, k, q_offset, out_dtype, scale)
        pg = None
    kind_code = HS_IDX_TOKEN if kind == "token" else HS_IDX_BLOCK
    cap = idx.shape[-1]
    keys = cap if kind_code == HS_IDX_TOKEN else cap * block
    sw = None
    window = 0
    keep = []
    if swa is not None:
        kl, vl, gate, window = swa
        loc_shape = ((q.shape[0], int(local_ring)) + tuple(k.shape[2:]) if local_ring
                     else (q.shape[0], desc.kv_len) + tuple(k.shape[2:]))
        _need(kl, "k_local", dev, dtype=q.dtype, shape=loc_shape)
        _need(vl, "v_local", dev, dtype=q.dtype, shape=loc_shape)
        _need(gate, "gate_logits", dev, dtype=torch.float32,
              shape=tuple(q.shape[:3]) + ((2, q.shape[3]) if gate_ch else (2,)))
        sw = SwaBranch(kl.data_ptr(), vl.data_ptr(), gate.data_ptr(), int(window))
        keep = [kl, vl, gate]
    o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = (torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=dev)
           if want_lse else None)
    ws, n = workspace(HS_OP_SPARSE_ATTN, desc, keys, window, device=dev)
    if (sink is None and sink_local is None and out_gate is None and not local_ring and pg is None
            and not gate_ch):
        _check(lib().hs_sparse_attn_gather(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                           kind_code, _ptr(idx), _ptr(count), int(cap),
                                           int(block),
                                           ctypes.byref(sw) if sw is not None else None, _ptr(o),
                                           _ptr(lse), _ptr(ws), n, _stream(dev)),
               "hs_sparse_attn_gather")
    else:
        Hq = q.shape[2]
        for t, nm, shp in ((sink, "sink", (Hq,)), (sink_local, "sink_local", (Hq,)),
                           (out_gate, "out_gate",
                            tuple(q.shape[:3]) + ((q.shape[3],) if gate_ch else ()))):
            if t is not None:
                _need(t, nm, dev, dtype=torch.float32, shape=shp)
        opts = SparseOpts(*(t.data_ptr() if t is not None else None
                            for t in (sink, sink_local, out_gate)), int(local_ring), gate_ch)
        _check(lib().hs_sparse_attn_gather_paged(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                                 ctypes.byref(pg) if pg is not None else None,
                                                 kind_code, _ptr(idx), _ptr(count), int(cap),
                                                 int(block),
                                                 ctypes.byref(sw) if sw is not None else None,
                                                 ctypes.byref(opts), _ptr(o), _ptr(lse),
                                                 _ptr(ws), n, _stream(dev)),
               "hs_sparse_attn_gather_paged")
    del keep
    return o, lse


def sparse_attn_gather_noalloc(q, k, v, idx, count, o, lse=None, kind="token", block=64,
                               swa=None, q_offset=None, scale=None):
    """hs_sparse_attn_gather_noalloc: the sparse layer without a workspace, writing into the
    caller's o [B,Tq,Hq,d] (and lse [B,Hq,Tq] fp32 when given).  Allocates nothing."""
    dev = q.device
    _need(q, "q", dev)
    _need(k, "k", dev, dtype=q.dtype)
    _need(v, "v", dev, dtype=q.dtype)
    _need(idx, "idx", dev, dtype=torch.int32)
    _need(count, "count", dev, dtype=torch.int32, shape=idx.shape[:3])
    _need(o, "o", dev, shape=q.shape)
    desc = make_desc(q, k, q_offset, o.dtype, scale)
    if lse is not None:
        _need(lse, "lse", dev, dtype=torch.float32, shape=(q.shape[0], q.shape[2], q.shape[1]))
    sw = None
    if swa is not None:
        kl, vl, gate, window = swa
        loc_shape = (q.shape[0], desc.kv_len) + tuple(k.shape[2:])
        _need(kl, "k_local", dev, dtype=q.dtype, shape=loc_shape)
        _need(vl, "v_local", dev, dtype=q.dtype, shape=loc_shape)
        _need(gate, "gate_logits", dev, dtype=torch.float32, shape=tuple(q.shape[:3]) + (2,))
        sw = SwaBranch(kl.data_ptr(), vl.data_ptr(), gate.data_ptr(), int(window))
    kind_code = HS_IDX_TOKEN if kind == "token" else HS_IDX_BLOCK
    _check(lib().hs_sparse_attn_gather_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                               kind_code, _ptr(idx), _ptr(count),
                                               int(idx.shape[-1]), int(block),
                                               ctypes.byref(sw) if sw is not None else None,
                                               _ptr(o), _ptr(lse), _stream(dev)),
           "hs_sparse_attn_gather_noalloc")
    return o, lse
