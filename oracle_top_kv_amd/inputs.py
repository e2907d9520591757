"""Seeded synthetic inputs and the workload table.

This module only draws random tensors and plants needles; it holds none of the attention,
scoring or selection arithmetic.  Both the GPU path and the CPU oracle consume the tensors it
returns (the oracle through ``.float().cpu().numpy()`` of the very same values).

Random draws: ``torch.randn`` / ``torch.randperm`` / ``torch.rand`` from a ``torch.Generator``
seeded per (workload seed, tensor role), then rounded once to the workload dtype (round to
nearest even for bf16).  The same seed on the same device type gives the same tensor.

Needles stand in for the retrieval-style peaked attention the pages' long-context workloads
exercise: a needle key is planted so that one chosen query head sees a large logit
a* = q.k / sqrt(d) at a position outside the forced local window, where only the top-k selection
can find it.
"""
from dataclasses import dataclass, replace
from typing import Dict, Optional

import torch

ROLE = {"q": 1, "k": 2, "v": 3, "k_loc": 4, "v_loc": 5, "gate": 6, "needle_pos": 7,
        "needle_amp": 8, "q_sparse": 100}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    kv_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"
    k_global: int = 1024
    window: int = 128
    n_sparse: int = 1
    block: int = 64
    n_blocks: int = 16
    needles: int = 0  # needles per (batch, kv head)
    needle_logit: float = 8.0
    cluster: int = 1  # consecutive positions per needle cluster (1 = single needles)
    needle_logit_hi: Optional[float] = None  # if set, a* ~ U[needle_logit, needle_logit_hi]
    seed: int = 1234

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def q_offset(self):
        return self.kv_len - self.q_len

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def shrink(self, **kw):
        return replace(self, **kw)


# Shapes of the pages' two model families (7B dense: 32 query / 8 KV heads; 80B-A3B MoE:
# 64 query / 4 KV heads; head dim 128; k = 1024, w = 128, 64-token blocks, 16 blocks).
WORKLOADS: Dict[str, Workload] = {
    # tiny causal prefill, fp32, correctness only
    "tiny_prefill_f32": Workload("tiny_prefill_f32", 1, 512, 512, 4, 1, 64, "f32",
                                 k_global=64, window=16, n_sparse=1, seed=101),
    # 7B-shaped decode at 32k context with 16 needles per KV head, 1 full + 3 sparse layers
    "decode_7b_32k": Workload("decode_7b_32k", 8, 1, 32768, 32, 8, 128, "bf16",
                              n_sparse=3, needles=16, needle_logit=8.0, seed=202),
    # 80B-shaped prefill chunk: 4096 queries appended to a 131072-token cache, 11 sparse layers
    "prefill_80b_128k": Workload("prefill_80b_128k", 1, 4096, 135168, 64, 4, 128, "bf16",
                                 n_sparse=11, seed=303),
    # 80B-shaped decode at 2^20 context, 16 clusters x 16 needles per KV head, 11 sparse layers
    "decode_80b_1m": Workload("decode_80b_1m", 4, 1, 1 << 20, 64, 4, 128, "bf16",
                              n_sparse=11, needles=16, cluster=16, needle_logit=6.0,
                              needle_logit_hi=10.0, seed=404),
    # HySparse block variant at 64k, gated sliding-window branch with its own K'/V'
    "block_7b_64k": Workload("block_7b_64k", 4, 65536, 65536, 32, 8, 128, "bf16",
                             n_sparse=1, seed=505),
    # HySparse2's own attention shape (MQA: 64 query heads on one KV head, d 256) in decode at
    # 32k context, 16 needles, 1 full + 3 sparse layers
    "decode_mqa256_32k": Workload("decode_mqa256_32k", 8, 1, 32768, 64, 1, 256, "bf16",
                                  n_sparse=3, needles=16, needle_logit=8.0, seed=606),
    # the same head shape in prefill: a 4096-query chunk appended to a 131072-token cache
    "prefill_mqa256_128k": Workload("prefill_mqa256_128k", 1, 4096, 135168, 64, 1, 256, "bf16",
                                    n_sparse=1, seed=707),
}


def _gen(wl: Workload, role: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + role)
    return g


def normal(shape, wl: Workload, role: int, device, dtype=None) -> torch.Tensor:
    """N(0,1) draws rounded once to ``dtype`` (default: the workload dtype)."""
    dtype = wl.torch_dtype if dtype is None else dtype
    x = torch.randn(shape, generator=_gen(wl, role, device), device=device, dtype=torch.float32)
    return x.to(dtype)


def _needle_positions(wl: Workload, gen: torch.Generator, device):
    """Per (b, u): start positions of the needle clusters, all inside 0 .. Tk-w-1 and pairwise
    non-overlapping (sorted distinct draws, then spread by the cluster length)."""
    span = wl.kv_len - wl.window - wl.needles * wl.cluster + 1
    assert span >= wl.needles, "context too short for the needles"
    starts = torch.empty(wl.batch, wl.n_kv_heads, wl.needles, dtype=torch.long)
    for b in range(wl.batch):
        for u in range(wl.n_kv_heads):
            pick = torch.randperm(span, generator=gen)[:wl.needles].sort().values
            starts[b, u] = pick + torch.arange(wl.needles) * wl.cluster
    return starts.to(device)


def plant_needles(wl: Workload, q: torch.Tensor, k: torch.Tensor) -> Dict[str, torch.Tensor]:
    """Overwrite needle keys in ``k`` (in place) so that head h_n = u*g + (n mod g) of the last
    query row sees the logit a*:  k = a* sqrt(d) q / |q|^2, rounded to the key dtype.
    Returns the planted positions [B, Hkv, needles*cluster] and the target heads."""
    if wl.needles == 0:
        return {}
    cpu = torch.device("cpu")
    gpos = _gen(wl, ROLE["needle_pos"], cpu)
    starts = _needle_positions(wl, gpos, cpu)
    if wl.needle_logit_hi is None:
        amp = torch.full((wl.batch, wl.n_kv_heads, wl.needles), wl.needle_logit)
    else:
        amp = wl.needle_logit + (wl.needle_logit_hi - wl.needle_logit) * torch.rand(
            (wl.batch, wl.n_kv_heads, wl.needles), generator=_gen(wl, ROLE["needle_amp"], cpu))
    g, d = wl.group, wl.head_dim
    qlast = q[:, -1].float()  # [B, Hq, d]
    positions = torch.empty(wl.batch, wl.n_kv_heads, wl.needles * wl.cluster, dtype=torch.long)
    heads = torch.empty(wl.batch, wl.n_kv_heads, wl.needles, dtype=torch.long)
    for b in range(wl.batch):
        for u in range(wl.n_kv_heads):
            for n in range(wl.needles):
                h = u * g + (n % g)
                qh = qlast[b, h]
                key = (float(amp[b, u, n]) * d ** 0.5) * qh / (qh * qh).sum()
                p0 = int(starts[b, u, n])
                k[b, p0:p0 + wl.cluster, u, :] = key.to(k.dtype)
                positions[b, u, n * wl.cluster:(n + 1) * wl.cluster] = torch.arange(
                    p0, p0 + wl.cluster)
                heads[b, u, n] = h
    return {"needle_pos": positions, "needle_head": heads}


def make_inputs(wl: Workload, device="cpu", n_sparse: Optional[int] = None,
                block_variant: bool = False) -> Dict[str, torch.Tensor]:
    """All inputs of one hot-path pass: the full layer's Q, K, V; one own Q' per sparse layer;
    for the block variant also the sparse layer's own K', V' and the gate logits."""
    device = torch.device(device)
    B, Tq, Tk, Hq, Hkv, d = (wl.batch, wl.q_len, wl.kv_len, wl.n_q_heads, wl.n_kv_heads,
                             wl.head_dim)
    out: Dict[str, torch.Tensor] = {}
    out["q"] = normal((B, Tq, Hq, d), wl, ROLE["q"], device)
    out["k"] = normal((B, Tk, Hkv, d), wl, ROLE["k"], device)
    out["v"] = normal((B, Tk, Hkv, d), wl, ROLE["v"], device)
    out.update(plant_needles(wl, out["q"], out["k"]))
    ns = wl.n_sparse if n_sparse is None else n_sparse
    out["q_sparse"] = [normal((B, Tq, Hq, d), wl, ROLE["q_sparse"] + i, device)
                       for i in range(ns)]
    if block_variant:
        out["k_loc"] = normal((B, Tk, Hkv, d), wl, ROLE["k_loc"], device)
        out["v_loc"] = normal((B, Tk, Hkv, d), wl, ROLE["v_loc"], device)
        out["gate"] = normal((B, Tq, Hq, 2), wl, ROLE["gate"], device, dtype=torch.float32)
    return out


def random_token_sets(batch: int, n_kv_heads: int, kv_len: int, k_global: int, window: int,
                      seed: int, device="cpu"):
    """Index sets of the token-sparse layer's shape for one decode query per (b, u) without running
    the selection: k_global distinct positions drawn uniformly from 0 .. kv_len-window-1, sorted,
    followed by the window kv_len-window .. kv_len-1.  Returns (idx int32 [B, 1, Hkv, k+w],
    count int32 [B, 1, Hkv]).  Used to time the gather kernel over many batch sizes."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    r = torch.rand(batch, n_kv_heads, kv_len - window, device=device, generator=g)
    top = r.topk(k_global, dim=-1).indices.sort(dim=-1).values.to(torch.int32)
    win = torch.arange(kv_len - window, kv_len, device=device, dtype=torch.int32)
    idx = torch.cat([top, win.expand(batch, n_kv_heads, window)], dim=-1)
    idx = idx.reshape(batch, 1, n_kv_heads, k_global + window).contiguous()
    cnt = torch.full((batch, 1, n_kv_heads), k_global + window, dtype=torch.int32, device=device)
    return idx, cnt


def to_numpy_f32(x: torch.Tensor):
    """Exact float32 copy on the host (bf16 widens exactly)."""
    return x.detach().float().cpu().numpy()
