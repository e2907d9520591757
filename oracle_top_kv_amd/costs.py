"""Algorithmic work of the hot path (bytes that must move, flops that must be done).

These are the figures the benchmark divides by measured time; they count what the method
requires, not what a kernel happens to read.  The cost-model formulas of the pages (KV capacity,
compute and read ratios) are included so that tests can pin the per-query budget constants to the
worked numbers printed there:
  [P2 "HySparse hybrid sparse attention (part 1)", pinghaoyang.com.cn, section "Cost model"
   and section "How cross-layer KV cache reuse works"].
"""


def kv_bytes_full_layer(batch, T, n_kv_heads, head_dim, bytes_per_elem):
    """K and V of one full-attention layer: 2 b T h_kv d s (M_full for one layer)."""
    return 2 * batch * T * n_kv_heads * head_dim * bytes_per_elem


def kv_capacity_ratio(F, S, T, w):
    """rho_M = (F T + S w) / (L T) with L = F + S."""
    return (F * T + S * w) / ((F + S) * T)


def prefill_compute_ratio(F, S, T, k, w):
    """rho_C ~ F/L + (S/L)(k+w)/T."""
    L = F + S
    return F / L + (S / L) * (k + w) / T


def decode_token_reads(F, S, T, k, w):
    """Token-KV positions read per decode step: F T + S (k + w)."""
    return F * T + S * (k + w)


def block_score_elements(T, B):
    """Elements of one head's block-score matrix if it were stored: T x ceil(T / B)."""
    return T * ((T + B - 1) // B)


def causal_pairs(q_len, kv_len):
    """Number of (query, key) pairs with key <= query position, queries at the last q_len
    positions of a kv_len context."""
    q0 = kv_len - q_len
    # sum_{t=q0}^{kv_len-1} (t + 1)
    return (q0 + 1 + kv_len) * q_len // 2


def index_set_size(t, k_global, window):
    """|I_t| = min(t + 1, k_global + window)."""
    return min(t + 1, k_global + window)


# ---- per-call algorithmic work of the library's entry points ------------------------------

def full_attn_flops(wl):
    """4 d flops per causal (query head, key) pair: q.k and p.v."""
    return 4 * wl.head_dim * wl.batch * wl.n_q_heads * causal_pairs(wl.q_len, wl.kv_len)


def full_attn_kv_bytes(wl, elem_bytes=2):
    """Decode-style lower bound: every K and V row of each (b, u) up to the last query read once."""
    return 2 * wl.batch * wl.kv_len * wl.n_kv_heads * wl.head_dim * elem_bytes


def score_flops(wl):
    """Logit recompute of the score pass: 2 d flops per causal (query head, key) pair."""
    return 2 * wl.head_dim * wl.batch * wl.n_q_heads * causal_pairs(wl.q_len, wl.kv_len)


def score_k_bytes(wl, elem_bytes=2):
    """Decode-style lower bound for the score pass: every K row read once."""
    return wl.batch * wl.kv_len * wl.n_kv_heads * wl.head_dim * elem_bytes


def token_gather_bytes(wl, elem_bytes=2):
    """K and V rows of every (b, t, u) index set: sum over query rows of |I_t| * 2 d s."""
    total = 0
    q0 = wl.kv_len - wl.q_len
    cap = wl.k_global + wl.window
    # |I_t| = min(t+1, cap) summed over t = q0 .. kv_len-1
    full = max(0, wl.kv_len - max(q0, cap - 1))  # rows with t + 1 >= cap
    total += full * cap
    lo, hi = q0, min(wl.kv_len, cap - 1)  # rows with t + 1 < cap: t = lo .. hi-1
    if hi > lo:
        total += (lo + 1 + hi) * (hi - lo) // 2
    return total * wl.batch * wl.n_kv_heads * 2 * wl.head_dim * elem_bytes


def block_gather_bytes(wl, elem_bytes=2):
    """HySparse sparse layer: n_blocks * B rows of the shared K, V plus w rows of the layer's own
    K', V' per (b, t, u) (upper bound at full blocks and a full window)."""
    rows = wl.n_blocks * wl.block + wl.window
    return wl.batch * wl.q_len * wl.n_kv_heads * rows * 2 * wl.head_dim * elem_bytes


def sparse_flops(wl):
    """Token-sparse layer: 4 d flops (QK and PV) per (query head, selected key)."""
    return 4 * wl.head_dim * wl.n_q_heads * (token_gather_bytes(wl) // (2 * wl.head_dim * 2 * wl.n_kv_heads))


def logit_bytes(wl):
    """Logits kept by full attention for the selections: one fp32 per (b, t, query head, key)."""
    return 4 * wl.batch * wl.q_len * wl.n_q_heads * wl.kv_len
