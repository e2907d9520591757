"""Python access to the CPU oracle (oracle/hs_oracle.c, IEEE double).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, by ``__graft_entry__.smoke()`` and by the
benchmark's CPU-baseline leg; the product package ``oracle_top_kv_amd`` never imports it.

Arrays are numpy, C-contiguous.  Float inputs are float32 holding exactly the values the GPU
sees; outputs are float64.  Shapes follow hs_oracle.h:
  q, o: [B, Tq, Hq, d]   k, v: [B, Tk, Hkv, d]   lse: [B, Hq, Tq]
  idx: [B, Tq, Hkv, cap] (int32, ascending, -1 padded)   count: [B, Tq, Hkv]
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_offset", ctypes.c_int64),
                ("scale", ctypes.c_double)]


def lib():
    """Load libhs_oracle.so, compiling it with gcc first if it is not there.  The environment
    variable HS_ORACLE_LIB points at another build (used by the mutation test, which plants
    mistakes in a copy of the source to show that the pins catch them)."""
    global _lib
    if _lib is None:
        path = os.environ.get("HS_ORACLE_LIB", _build.SO)
        if path == _build.SO and not os.path.exists(path):
            _build.build()
        _lib = ctypes.CDLL(path)
        _lib.orc_set_threads.argtypes = [ctypes.c_int]
    return _lib


def set_threads(n):
    return lib().orc_set_threads(int(n))


def threads():
    return lib().orc_threads()


def _f32(x):
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _f64(x):
    a = np.ascontiguousarray(x, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _i32(x):
    a = np.ascontiguousarray(x, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _shape(q, k, q_offset, scale=None):
    """scale: the logit scale tau (None: 1/sqrt(d))."""
    B, Tq, Hq, d = q.shape
    Bk, Tk, Hkv, dk = k.shape
    assert B == Bk and d == dk, "q/k shapes disagree"
    if q_offset is None:
        q_offset = Tk - Tq
    return Shape(B, Tq, Tk, Hq, Hkv, d, int(q_offset), 0.0 if scale is None else float(scale))


def _rows(rows):
    if rows is None:
        return None, None, 0
    r, p = _i32(rows)
    return r, p, len(r)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def full_attention(q, k, v, q_offset=None, rows=None, scale=None):
    """Exact causal GQA attention. Returns (o float64 [B,Tq,Hq,d], lse float64 [B,Hq,Tq]).
    With ``rows`` only those query rows are computed (others are NaN)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    o = np.full(q.shape, np.nan)
    lse = np.full((s.batch, s.n_q_heads, s.q_len), np.nan)
    rr, rp, nr = _rows(rows)
    _check(lib().orc_full_attention(ctypes.byref(s), qp, kp, vp, o.ctypes.data_as(ctypes.c_void_p),
                                    lse.ctypes.data_as(ctypes.c_void_p), rp, nr), "full_attention")
    return o, lse


def logit_row(q, k, b, j, h, q_offset=None, scale=None):
    """Scaled logits a_{t,i} = q.k_i / sqrt(d), i = 0..t, of one (b, j, h)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    t = s.q_offset + j
    a = np.empty(t + 1)
    _check(lib().orc_logit_row(ctypes.byref(s), qp, kp, b, j, h,
                               a.ctypes.data_as(ctypes.c_void_p)), "logit_row")
    return a


def prob_row(q, k, b, j, h, lse=None, q_offset=None, scale=None):
    """Per-head normalized probabilities p_{t,i}, i = 0..t, of one (b, j, h)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    t = s.q_offset + j
    p = np.empty(t + 1)
    lp = None
    if lse is not None:
        lse, lp = _f64(lse)
    _check(lib().orc_prob_row(ctypes.byref(s), qp, kp, lp, b, j, h,
                              p.ctypes.data_as(ctypes.c_void_p)), "prob_row")
    return p


def token_score_row(q, k, lse, b, j, u, q_offset=None, scale=None):
    """Token scores max_{h in group u} p^h_{t,i}, i = 0..t, of one (b, j, u)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    t = s.q_offset + j
    out = np.empty(t + 1)
    lp = None
    if lse is not None:
        lse, lp = _f64(lse)
    _check(lib().orc_token_score_row(ctypes.byref(s), qp, kp, lp, b, j, u,
                                     out.ctypes.data_as(ctypes.c_void_p)), "token_score_row")
    return out


def token_topk(q, k, lse, k_global, window, cap=None, q_offset=None, rows=None, scale=None):
    """Forced window plus top-k_global outside it. Returns (idx int32 [B,Tq,Hkv,cap], count)."""
    s = _shape(q, k, q_offset, scale)
    cap = k_global + window if cap is None else cap
    q, qp = _f32(q)
    k, kp = _f32(k)
    lp = None
    if lse is not None:
        lse, lp = _f64(lse)
    idx = np.full((s.batch, s.q_len, s.n_kv_heads, cap), -2, dtype=np.int32)
    cnt = np.full((s.batch, s.q_len, s.n_kv_heads), -2, dtype=np.int32)
    rr, rp, nr = _rows(rows)
    _check(lib().orc_token_topk(ctypes.byref(s), qp, kp, lp, int(k_global), int(window), int(cap),
                                idx.ctypes.data_as(ctypes.c_void_p),
                                cnt.ctypes.data_as(ctypes.c_void_p), rp, nr), "token_topk")
    return idx, cnt


def _opt_f32(x):
    if x is None:
        return None, None
    return _f32(x)


def masked_attention(q, k, v, idx, count, q_offset=None, rows=None, sink=None, out_gate=None,
                     scale=None):
    """Attention of q over k, v restricted to each row's index set (dense masked softmax).
    sink: [Hq] per-head sink logits in the denominator; out_gate: sigmoid output-gate logits,
    [B,Tq,Hq] (one per head) or [B,Tq,Hq,d] (one per channel).  Returns (o float64, lse float64;
    lse includes the sink)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    idx, ip = _i32(idx)
    count, cp = _i32(count)
    o = np.full(q.shape, np.nan)
    lse = np.full((s.batch, s.n_q_heads, s.q_len), np.nan)
    rr, rp, nr = _rows(rows)
    sk, skp = _opt_f32(sink)
    og, ogp = _opt_f32(out_gate)
    fn = lib().orc_masked_attention_ex
    if og is not None and og.ndim == q.ndim:
        fn = lib().orc_masked_attention_ch
    _check(fn(ctypes.byref(s), qp, kp, vp, ip, cp, int(idx.shape[-1]), skp, ogp,
              o.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p), rp, nr),
           "masked_attention")
    return o, lse


def block_score_row(q, k, lse, b, j, u, block, q_offset=None, scale=None):
    """Group-max block scores of the causal blocks 0..floor(t/B) of one (b, j, u)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    t = s.q_offset + j
    out = np.empty(t // block + 1)
    lp = None
    if lse is not None:
        lse, lp = _f64(lse)
    _check(lib().orc_block_score_row(ctypes.byref(s), qp, kp, lp, b, j, u, int(block),
                                     out.ctypes.data_as(ctypes.c_void_p)), "block_score_row")
    return out


def block_topk(q, k, lse, block, n_blocks, q_offset=None, rows=None, scale=None):
    """Top n_blocks causal blocks. Returns (blk_idx int32 [B,Tq,Hkv,n_blocks] ascending, count)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    lp = None
    if lse is not None:
        lse, lp = _f64(lse)
    idx = np.full((s.batch, s.q_len, s.n_kv_heads, n_blocks), -2, dtype=np.int32)
    cnt = np.full((s.batch, s.q_len, s.n_kv_heads), -2, dtype=np.int32)
    rr, rp, nr = _rows(rows)
    _check(lib().orc_block_topk(ctypes.byref(s), qp, kp, lp, int(block), int(n_blocks),
                                idx.ctypes.data_as(ctypes.c_void_p),
                                cnt.ctypes.data_as(ctypes.c_void_p), rp, nr), "block_topk")
    return idx, cnt


def gated_block_swa(q, k, v, blk_idx, count, block, k_loc, v_loc, window, gate, q_offset=None,
                    rows=None, sink=None, sink_loc=None, out_gate=None, scale=None):
    """HySparse sparse layer.  gate: the two branch-gate logits (zG, zL), [B,Tq,Hq,2] (per head)
    or [B,Tq,Hq,2,d] (per channel); sink / sink_loc: [Hq] sink logits of the two branches;
    out_gate: sigmoid output-gate logits on the gated sum, [B,Tq,Hq] or [B,Tq,Hq,d] (per-channel
    gates come as a pair: both gate and out_gate per channel, or out_gate None).  Returns
    (o, o_glob, o_loc), all float64 [B,Tq,Hq,d] (o_glob, o_loc: the normalized branches before
    the gates)."""
    s = _shape(q, k, q_offset, scale)
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    kl, klp = _f32(k_loc)
    vl, vlp = _f32(v_loc)
    gt, gp = _f32(gate)
    bi, bp = _i32(blk_idx)
    cnt, cp = _i32(count)
    o = np.full(q.shape, np.nan)
    og = np.full(q.shape, np.nan)
    ol = np.full(q.shape, np.nan)
    rr, rp, nr = _rows(rows)
    sk, skp = _opt_f32(sink)
    sl, slp = _opt_f32(sink_loc)
    ogt, ogtp = _opt_f32(out_gate)
    per_channel = gt.ndim == q.ndim + 1
    if ogt is not None and per_channel != (ogt.ndim == q.ndim):
        raise ValueError("gated_block_swa: gate and out_gate must both be per head or per channel")
    fn = lib().orc_gated_block_swa_ch if per_channel else lib().orc_gated_block_swa_ex
    _check(fn(ctypes.byref(s), qp, kp, vp, bp, cp, int(bi.shape[-1]), int(block), klp, vlp,
              int(window), gp, skp, slp, ogtp, o.ctypes.data_as(ctypes.c_void_p),
              og.ctypes.data_as(ctypes.c_void_p), ol.ctypes.data_as(ctypes.c_void_p), rp, nr),
           "gated_block_swa")
    return o, og, ol
