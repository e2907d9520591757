"""Benchmark of the hot path on one MI355X.

One step = one pass of every stage of the hot path over one batch of the 7B-shaped decode
workload (batch 8, 32768-token context, 32 query / 8 KV heads, d = 128, bf16, 16 needles per KV
head):
  full attention with LSE -> token oracle top-k (1024 + window 128) -> 3 token-sparse layers
  (each with its own Q') -> block scores + top-16 blocks -> a block-sparse layer with its gated
  sliding-window branch (own K', V').
Inputs are generated on the GPU before timing and stay resident in HBM.  In a model the layers
between two sparse layers (feed-forward weights, other layers' caches) stream gigabytes through
the GPU's caches, so every sparse layer of the step runs cold: a 1 GiB read of another buffer
(not counted in any stage) evicts L2 and the 256 MB last-level cache right before each one.

Prints ONE JSON line.  `value` is the metric's sparse half: gathered K+V bytes of the step's
token-sparse layers (|I_t| rows of K and V per (b, t, u): 37,748,736 B per layer) over their
event-timed durations, i.e. cold-cache sparse-attention GB/s.  `roofline` is that layer against
8 TB/s.  The step's other stages, the prefill legs (full attention + top-k TFLOP/s, the metric's
other half), the block workload at its own shape and the measured ceilings follow as fields.
Per-stage times come from HIP events recorded on torch's current stream, which is the stream
the library launches on.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn gathered KV GB/s + full-attn+topk prefill TFLOP/s, % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
SCRUB_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_7b_32k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU-oracle baselines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 80B prefill-chunk leg")
    ap.add_argument("--no-block-prefill", action="store_true",
                    help="skip the 64k block workload's prefill legs (scoring and sparse layer)")
    ap.add_argument("--no-long-decode", action="store_true",
                    help="skip the 2^20-context decode leg")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the batch sweep of the token-sparse decode layer")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a device copy of MIB MiB (the reference kernel of the HBM "
                         "counter scaling) and exit")
    return ap.parse_args()


def copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_MiB": mib}), flush=True)


def rate(byts, ms):
    return byts / (ms * 1e-3) / 1e9


class Probes:
    """The measurement kernels of oracle_top_kv_amd/probes/ceilings.hip (libhs_probes.so): a
    contiguous HBM read and a gather of random K / V rows, on torch's current stream.  The
    read doubles as the cache scrub: reading 1 GiB replaces the contents of L2 and of the 256 MB
    last-level cache with clean lines, as the weights read by a model's other layers would."""

    def __init__(self, torch):
        import ctypes
        path = os.path.join(ROOT, "oracle_top_kv_amd", "libhs_probes.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.probe_read_stream.argtypes = [vp, sz, vp, vp]
        L.probe_read_stream_out_words.argtypes = [sz]
        L.probe_read_stream_out_words.restype = sz
        L.probe_row_gather.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
        L.probe_row_gather_out_words.argtypes = [i32, i32, i32]
        L.probe_row_gather_out_words.restype = sz
        self.L, self.torch, self.ctypes = L, torch, ctypes
        self.scrub_buf = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda:0")
        self.scrub_out = torch.empty(L.probe_read_stream_out_words(SCRUB_BYTES),
                                     dtype=torch.int32, device="cuda:0")

    def _stream(self):
        return self.ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def read(self, buf, out):
        rc = self.L.probe_read_stream(buf.data_ptr(), buf.numel() * buf.element_size(),
                                      out.data_ptr(), self._stream())
        if rc:
            raise RuntimeError(f"probe_read_stream: HIP error {rc}")

    def scrub(self):
        self.read(self.scrub_buf, self.scrub_out)

    def gather(self, k, v, idx, out):
        B, T, Hkv, d = k.shape
        cap = idx.shape[-1]
        rc = self.L.probe_row_gather(k.data_ptr(), v.data_ptr(), idx.data_ptr(), B, T, Hkv, cap,
                                     d * k.element_size(), out.data_ptr(), self._stream())
        if rc:
            raise RuntimeError(f"probe_row_gather: HIP error {rc}")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(wl, device=dev, block_variant=True)
    q, k, v = x["q"], x["k"], x["v"]
    qs = x["q_sparse"]
    kl, vl, gate = x["k_loc"], x["v_loc"], x["gate"]
    probes = Probes(torch)
    torch.cuda.synchronize()

    stages = ["full_attn", "token_topk", "sparse_token", "block_topk", "sparse_block_swa"]
    n_ev = 3 + 2 * wl.n_sparse + 4

    def step(ev=None):
        """One pass of the hot path.  Events (when given): [0,1] full attention, [1,2] token
        top-k, then a pair around each sparse layer (after its scrub), then [.., ..] block top-k
        and a pair around the gated layer."""
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        o, lse = hs.full_attn_fwd(q, k, v)
        mark(1)
        idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
        mark(2)
        for l in range(wl.n_sparse):
            probes.scrub()
            mark(3 + 2 * l)
            hs.sparse_attn_gather(qs[l], k, v, idx, cnt, kind="token")
            mark(4 + 2 * l)
        i0 = 3 + 2 * wl.n_sparse
        mark(i0)
        bidx, bcnt = hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        mark(i0 + 1)
        probes.scrub()
        mark(i0 + 2)
        hs.sparse_attn_gather(qs[0], k, v, bidx, bcnt, kind="block", block=wl.block,
                              swa=(kl, vl, gate, wl.window))
        mark(i0 + 3)

    def stage_times(e):
        i0 = 3 + 2 * wl.n_sparse
        return {"full_attn": e[0].elapsed_time(e[1]), "token_topk": e[1].elapsed_time(e[2]),
                "sparse_token": [e[3 + 2 * l].elapsed_time(e[4 + 2 * l])
                                 for l in range(wl.n_sparse)],
                "block_topk": e[i0].elapsed_time(e[i0 + 1]),
                "sparse_block_swa": e[i0 + 2].elapsed_time(e[i0 + 3])}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, bracketed by synchronization, with per-stage events
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step(evs[s])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    per = [stage_times(e) for e in evs]
    layer_ms = sorted(t for p_ in per for t in p_["sparse_token"])  # every cold token layer
    stage_all = {n: sorted((sum(p_[n]) if n == "sparse_token" else p_[n]) for p_ in per)
                 for n in stages}
    stage_ms = {n: sum(v_) / len(v_) for n, v_ in stage_all.items()}

    # algorithmic bytes per stage
    b_full = costs.full_attn_kv_bytes(wl)                 # K and V read once
    b_score = costs.score_k_bytes(wl)                     # K read once per scoring pass
    b_tok = costs.token_gather_bytes(wl)                  # per sparse layer
    b_blk = costs.block_gather_bytes(wl)                  # per block-sparse + SWA layer
    stage_bytes = {"full_attn": b_full, "token_topk": b_score,
                   "sparse_token": wl.n_sparse * b_tok, "block_topk": b_score,
                   "sparse_block_swa": b_blk}
    step_bytes = sum(stage_bytes.values())
    layer_avg_ms = sum(layer_ms) / len(layer_ms)
    value = rate(b_tok, layer_avg_ms)  # cold token-sparse layers: total bytes / total time

    stages_out = {}
    for n in stages:
        gbs = rate(stage_bytes[n], stage_ms[n])
        v_ = stage_all[n]
        stages_out[n] = {"ms": round(stage_ms[n], 4), "median_ms": round(v_[len(v_) // 2], 4),
                         "min_ms": round(v_[0], 4), "GB_per_s": round(gbs, 1),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 3)}
    stages_out["sparse_token"].update(
        {"per_layer_gathered_bytes": b_tok, "per_layer_avg_us": round(layer_avg_ms * 1e3, 2),
         "per_layer_median_us": round(layer_ms[len(layer_ms) // 2] * 1e3, 2),
         "per_layer_min_us": round(layer_ms[0] * 1e3, 2), "cache": "cold (scrub before each)"})
    stages_out["sparse_block_swa"]["cache"] = "cold (scrub before)"
    fa_gbs = rate(b_full, stage_ms["full_attn"])

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "kv_len": wl.kv_len,
                   "q_len": wl.q_len, "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "k_global": wl.k_global, "window": wl.window,
                   "sparse_layers": wl.n_sparse, "block": wl.block, "n_blocks": wl.n_blocks,
                   "needles_per_kv_head": wl.needles},
        "value_is": "gathered K+V bytes of the step's token-sparse layers / their event time, "
                    "each layer cold (after a 1 GiB read of another buffer)",
        "roofline": {"bound": "hbm",
                     "kernel": "token-sparse decode layer (row_attn_kernel over the index set "
                               "+ combine_kernel), cold cache",
                     "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "algorithmic_bytes": b_tok,
                     "traffic": counter_traffic(wl.name, "sparse_token")},
        "roofline_full_attn": {"bound": "hbm", "kernel": "full-attention decode call "
                                                         "(row_attn_kernel + combine_kernel)",
                               "achieved": round(fa_gbs, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(fa_gbs / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes": b_full,
                               "traffic": counter_traffic(wl.name, "full_attn")},
        "step": {"bytes": step_bytes,
                 "GB_per_s_stages": round(rate(step_bytes, sum(stage_ms.values())), 1),
                 "ms_stages": round(sum(stage_ms.values()), 4),
                 "scrub_ms": round(ms_step - sum(stage_ms.values()), 4),
                 "note": "step bytes / the stages' event time (the scrubs excluded)"},
        "stages": stages_out,
    }
    out["step_warm_graph"] = warm_steps(wl, x, hs, costs, args)
    out["step_paged"] = paged_step(wl, x, hs, args, out["step_warm_graph"]["stored_logits_ms"])
    peaks = measured_peaks(x, wl, probes)
    out["measured_peaks"] = peaks
    out["roofline"]["frac_of_measured_gather"] = round(value / peaks["row_gather_GB_per_s"], 4)
    out["roofline_full_attn"]["frac_of_measured_read"] = round(
        fa_gbs / peaks["read_stream_GB_per_s"], 4)
    # the oracle baselines run later on the same inputs (kept on the GPU until then)
    cpu_x = None if args.no_cpu_baseline else {n: x[n] for n in
                                               ("q", "k", "v", "k_loc", "v_loc", "gate",
                                                "q_sparse")}
    del x, q, k, v, qs, kl, vl, gate, probes
    torch.cuda.empty_cache()
    out["block_decode"] = block_decode_leg(args)
    gemm = peaks["gemm_bf16_TFLOP_per_s"]
    if not args.no_prefill:
        out["prefill"] = prefill_leg(args)
        out["prefill"]["full_attn_frac_of_measured_gemm"] = round(
            out["prefill"]["full_attn_tflops"] / gemm, 4)
        fa = out["prefill"]
        out["roofline_prefill"] = {"bound": "mfma", "kernel": "prefill full attention "
                                                             "(pf_attn_kernel), bf16",
                                   "achieved": fa["full_attn_tflops"], "peak": BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": fa["mfma_frac_full_attn"],
                                   "algorithmic_flops": costs.full_attn_flops(
                                       WORKLOADS["prefill_80b_128k"]), "traffic": None}
    if not args.no_block_prefill:
        out["block_prefill"] = block_prefill_leg(args)
    out["mqa256_decode"] = mqa256_leg(args)
    if not args.no_prefill:
        out["mqa256_prefill"] = mqa256_prefill_leg()
    if not args.no_long_decode:
        out["long_decode"] = long_decode_leg(args, cpu=not args.no_cpu_baseline)
    if not args.no_sweep:
        out["sparse_decode_sweep"] = sparse_sweep(wl)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_sparse(wl, cpu_x, args.cpu_seconds)
        out["cpu_baseline_step"] = cpu_baseline(wl, cpu_x, args.cpu_seconds)
        if not args.no_prefill:
            out["cpu_baseline_prefill"] = cpu_baseline_prefill(out.get("prefill"))
        if not args.no_block_prefill:
            out["cpu_baseline_block"] = cpu_baseline_block(out.get("block_prefill"))
    print(json.dumps(out), flush=True)


def warm_steps(wl, x, hs, costs, args):
    """The same step without scrubs (the sparse layers then read rows the previous layer left
    in cache), eager and replayed from a HIP graph, and the step with both selections reading
    the logits full attention kept instead of re-reading K.  The library allocates nothing,
    never synchronizes and zero-fills with kernels, so every call is capturable."""
    import torch

    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"]
    swa = (x["k_loc"], x["v_loc"], x["gate"], wl.window)

    def step():
        o, lse = hs.full_attn_fwd(q, k, v)
        idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
        for l in range(wl.n_sparse):
            hs.sparse_attn_gather(qs[l], k, v, idx, cnt, kind="token")
        bidx, bcnt = hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        hs.sparse_attn_gather(qs[0], k, v, bidx, bcnt, kind="block", block=wl.block, swa=swa)

    def step_logits():
        o, lse, lg = hs.full_attn_fwd_logits(q, k, v)
        idx, cnt = hs.oracle_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.k_global,
                                              wl.window)
        for l in range(wl.n_sparse):
            hs.sparse_attn_gather(qs[l], k, v, idx, cnt, kind="token")
        bidx, bcnt = hs.block_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.block,
                                               wl.n_blocks)
        hs.sparse_attn_gather(qs[0], k, v, bidx, bcnt, kind="block", block=wl.block, swa=swa)

    def eager_ms(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = eager_ms(step)
    ms_l = eager_ms(step_logits)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    ms_g = eager_ms(graph.replay)
    del graph
    b = (costs.full_attn_kv_bytes(wl) + 2 * costs.score_k_bytes(wl) +
         wl.n_sparse * costs.token_gather_bytes(wl) + costs.block_gather_bytes(wl))
    b_l = (costs.full_attn_kv_bytes(wl) + 3 * costs.logit_bytes(wl) +
           wl.n_sparse * costs.token_gather_bytes(wl) + costs.block_gather_bytes(wl))
    return {"ms": round(ms, 4), "graph_ms": round(ms_g, 4), "bytes": b,
            "GB_per_s": round(rate(b, ms), 1), "stored_logits_ms": round(ms_l, 4),
            "stored_logits_bytes": b_l, "stored_logits_GB_per_s": round(rate(b_l, ms_l), 1),
            "speedup_stored_logits": round(ms / ms_l, 3)}


def counter_traffic(workload, stage):
    """HBM bytes per launch of one stage's kernels from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading); None when that summary
    is missing, covers another workload or stage, or any kernel source it lists has changed
    since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    meta = json.loads(m.group(1))
    per = meta.get("traffic_bytes_per_launch")
    if meta.get("workload") != workload or not isinstance(per, dict) or stage not in per:
        return None
    for rel, digest in meta["sources_sha256"].items():
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != digest:
            return None
    return meta["traffic_bytes_per_launch"][stage]


def prefill_leg(args):
    """Full attention + token top-k + one token-sparse layer on the 80B-shaped prefill chunk
    (4096 queries appended to a 131072-token cache, 64/4 heads, d 128, bf16): TFLOP/s of the
    full-attention flops plus the score-recompute flops over the first two calls' time, of the
    full-attention flops alone, and the sparse layer's time with its logical gathered bytes
    (every query's index-set rows; neighbouring queries share most of them in cache)."""
    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS["prefill_80b_128k"]
    x = make_inputs(wl, device=torch.device("cuda:0"), n_sparse=1)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    for _ in range(2):
        _, lse = hs.full_attn_fwd(q, k, v)
        idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
        hs.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")
    torch.cuda.synchronize()
    reps = 5
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record()
        _, lse = hs.full_attn_fwd(q, k, v)
        ev[r][1].record()
        idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
        ev[r][2].record()
        hs.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")
        ev[r][3].record()
    torch.cuda.synchronize()
    t_fa = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    t_tk = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    t_sp = sum(e[2].elapsed_time(e[3]) for e in ev) / reps
    # the same two stages in one call: the selection starts at the tile-maximum bound
    _, _, idx1, cnt1 = hs.full_attn_topk(q, k, v, wl.k_global, wl.window)
    torch.cuda.synchronize()
    same = bool(torch.equal(idx1, idx) and torch.equal(cnt1, cnt))
    ev1 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for r in range(reps):
        ev1[r][0].record()
        hs.full_attn_topk(q, k, v, wl.k_global, wl.window)
        ev1[r][1].record()
    torch.cuda.synchronize()
    t_one = sum(e[0].elapsed_time(e[1]) for e in ev1) / reps
    paged = paged_prefill(wl, q, k, v, qs, idx, cnt, hs, reps)
    f_fa, f_sc = costs.full_attn_flops(wl), costs.score_flops(wl)
    tot = (f_fa + f_sc) / ((t_fa + t_tk) * 1e-3) / 1e12
    b_sp = costs.token_gather_bytes(wl)  # rows each (b, t, u) gathers (mostly from cache)
    f_sp = costs.sparse_flops(wl)
    return {"workload": wl.name, "full_attn_ms": round(t_fa, 3), "topk_ms": round(t_tk, 3),
            "full_attn_tflops": round(f_fa / (t_fa * 1e-3) / 1e12, 1),
            "topk_score_tflops": round(f_sc / (t_tk * 1e-3) / 1e12, 1),
            "full_attn_plus_topk_tflops": round(tot, 1),
            "one_call_full_attn_topk_ms": round(t_one, 3),
            "one_call_full_attn_topk_tflops": round((f_fa + f_sc) / (t_one * 1e-3) / 1e12, 1),
            "one_call_sets_identical": same,
            "useful_tflops": round(f_fa / ((t_fa + t_tk) * 1e-3) / 1e12, 1),
            "mfma_frac_full_attn": round(f_fa / (t_fa * 1e-3) / 2.5e15, 4),
            "sparse_layer_ms": round(t_sp, 3),
            "sparse_layer_logical_GB_per_s": round(b_sp / (t_sp * 1e-3) / 1e9, 1),
            "sparse_layer_tflops": round(f_sp / (t_sp * 1e-3) / 1e12, 1),
            "paged": dict(paged, vs_contiguous={
                "full_attn": round(paged["full_attn_ms"] / t_fa, 3),
                "topk": round(paged["topk_ms"] / t_tk, 3),
                "sparse_layer": round(paged["sparse_layer_ms"] / t_sp, 3)}),
            "peak_tflops": 2500.0, "reps": reps}


def paged_prefill(wl, q, k, v, qs, idx, cnt, hs, reps, page_size=64):
    """Full attention, token top-k and one token-sparse layer of a prefill chunk over a paged
    cache: K and V in shuffled 64-position pages behind a block table (the tiled attention and
    the streamed selection read each key tile from its page).  Checks that the index sets equal
    the contiguous calls' (idx, cnt)."""
    import torch

    B, T, Hkv, d = k.shape
    mp = (T + page_size - 1) // page_size
    g = torch.Generator().manual_seed(19)
    table = torch.randperm(B * mp, generator=g).view(B, mp).to(torch.int32)
    inv = torch.empty(B * mp, dtype=torch.long)
    inv[table.view(-1).long()] = torch.arange(B * mp)
    table, inv = table.cuda(), inv.cuda()

    def pool(t):
        p = t.view(B * mp, page_size, Hkv, d)  # logical page order (T is a multiple of 64)
        return p[inv].contiguous()              # physical page table[b, lp] holds page (b, lp)

    kp, vp = pool(k), pool(v)
    pages = (table, T)
    _, lse = hs.full_attn_fwd_paged(q, kp, vp, table, T)
    pi, pc = hs.oracle_topk(q, kp, lse, wl.k_global, wl.window, pages=pages)
    hs.sparse_attn_gather(qs, kp, vp, pi, pc, kind="token", pages=pages)
    torch.cuda.synchronize()
    same = bool(torch.equal(pi, idx) and torch.equal(pc, cnt))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record()
        _, lse = hs.full_attn_fwd_paged(q, kp, vp, table, T)
        ev[r][1].record()
        pi, pc = hs.oracle_topk(q, kp, lse, wl.k_global, wl.window, pages=pages)
        ev[r][2].record()
        hs.sparse_attn_gather(qs, kp, vp, pi, pc, kind="token", pages=pages)
        ev[r][3].record()
    torch.cuda.synchronize()
    t = [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / reps for i in range(3)]
    del kp, vp
    return {"page_size": page_size, "full_attn_ms": round(t[0], 3), "topk_ms": round(t[1], 3),
            "sparse_layer_ms": round(t[2], 3), "sets_identical_to_contiguous": same}


def mqa256_prefill_leg():
    """HySparse2's own head shape (MQA: 64 query heads on one KV head, d 256) in prefill: a
    4096-query chunk appended to a 131072-token cache.  Full attention on the tiled prefill
    kernel (128 rows per workgroup), token top-k per 16-head chunk with the exact chunk merge
    (no per-key score is stored), one token-sparse layer; TFLOP/s as in the 80B prefill leg."""
    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS["prefill_mqa256_128k"]
    x = make_inputs(wl, device=torch.device("cuda:0"), n_sparse=1)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    _, lse = hs.full_attn_fwd(q, k, v)
    idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
    hs.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")
    torch.cuda.synchronize()
    reps = 5
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record()
        _, lse = hs.full_attn_fwd(q, k, v)
        ev[r][1].record()
        idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
        ev[r][2].record()
        hs.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")
        ev[r][3].record()
    torch.cuda.synchronize()
    t_fa, t_tk, t_sp = (sum(e[i].elapsed_time(e[i + 1]) for e in ev) / reps for i in range(3))
    f_fa, f_sc = costs.full_attn_flops(wl), costs.score_flops(wl)
    del x, q, k, v, qs, lse, idx, cnt
    torch.cuda.empty_cache()
    return {"workload": wl.name, "full_attn_ms": round(t_fa, 3), "topk_ms": round(t_tk, 3),
            "full_attn_tflops": round(f_fa / (t_fa * 1e-3) / 1e12, 1),
            "mfma_frac_full_attn": round(f_fa / (t_fa * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "topk_score_tflops": round(f_sc / (t_tk * 1e-3) / 1e12, 1),
            "full_attn_plus_topk_tflops": round((f_fa + f_sc) / ((t_fa + t_tk) * 1e-3) / 1e12, 1),
            "sparse_layer_ms": round(t_sp, 3),
            "sparse_layer_logical_GB_per_s": round(rate(costs.token_gather_bytes(wl), t_sp), 1),
            "reps": reps}


def paged_step(wl, x, hs, args, ms_contiguous, page_size=64):
    """The stored-logits decode step on a paged cache: K and V in shuffled 64-position pages
    behind a block table, the window branch's own K', V' in a ring of `window` slots."""
    import torch

    B, T, Hkv, d = x["k"].shape
    mp = (T + page_size - 1) // page_size
    g = torch.Generator().manual_seed(17)
    table = torch.randperm(B * mp, generator=g).view(B, mp).to(torch.int32).cuda()
    inv = torch.empty(B * mp, dtype=torch.long)
    inv[table.view(-1).cpu().long()] = torch.arange(B * mp)
    inv = inv.cuda()

    def pool(t):
        p = t.view(B * mp, page_size, Hkv, d)  # logical page order (T is a multiple of 64)
        return p[inv].contiguous()              # physical page table[b, lp] holds page (b, lp)

    kp, vp = pool(x["k"]), pool(x["v"])
    ring = wl.window
    first = T - ring
    kl = torch.zeros((B, ring, Hkv, d), dtype=x["k"].dtype, device="cuda")
    vl = torch.zeros_like(kl)
    pos = torch.arange(first, T, device="cuda")
    kl[:, pos % ring] = x["k_loc"][:, first:]
    vl[:, pos % ring] = x["v_loc"][:, first:]
    pages = (table, T)
    qs = x["q_sparse"]

    def step():
        o, lse, lg = hs.full_attn_fwd_paged(x["q"], kp, vp, table, T, logits=True)
        idx, cnt = hs.oracle_topk_from_logits(lg, lse, Hkv, d, wl.k_global, wl.window)
        for l in range(wl.n_sparse):
            hs.sparse_attn_gather(qs[l], kp, vp, idx, cnt, kind="token", pages=pages)
        bidx, bcnt = hs.block_topk_from_logits(lg, lse, Hkv, d, wl.block, wl.n_blocks)
        hs.sparse_attn_gather(qs[0], kp, vp, bidx, bcnt, kind="block", block=wl.block,
                              swa=(kl, vl, x["gate"], wl.window), local_ring=ring, pages=pages)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    del kp, vp, kl, vl
    return {"ms_per_step": round(ms, 4), "page_size": page_size, "local_ring": ring,
            "vs_contiguous_stored_logits": round(ms / ms_contiguous, 3)}


def measured_peaks(x, wl, probes):
    """Ceilings measured on this GPU: a 1 GiB device copy (bytes read plus written per second),
    a contiguous read of 2 GiB (the probe kernel, non-temporal loads), a gather of random K and V
    rows of the benchmark's own cache by the probe kernel (the token-sparse layer's pattern and
    size: 1024 random positions below T - 128 plus the last 128 per (b, u); cold, after the
    scrub, and warm) and a large bf16 GEMM (the GEMM library; dense MFMA TFLOP/s)."""
    import torch

    from oracle_top_kv_amd.inputs import random_token_sets

    def timed(fn, reps, cold=False):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            if cold:
                probes.scrub()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(ts)[reps // 2]

    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    t_copy = timed(lambda: b.copy_(a), 10)
    del a, b
    r = torch.ones(2 * n, dtype=torch.float32, device="cuda:0")
    ro = torch.empty(probes.L.probe_read_stream_out_words(8 * n), dtype=torch.int32,
                     device="cuda:0")
    t_read = timed(lambda: probes.read(r, ro), 10)
    del r, ro
    B, T, Hkv, d = x["k"].shape
    idx, _ = random_token_sets(B, Hkv, T, wl.k_global, wl.window, seed=77, device="cuda:0")
    idx = idx.view(B, Hkv, -1).contiguous()
    go = torch.empty(probes.L.probe_row_gather_out_words(B, Hkv, idx.shape[-1]),
                     dtype=torch.int32, device="cuda:0")
    g_bytes = B * Hkv * idx.shape[-1] * 2 * d * x["k"].element_size()
    t_gw = timed(lambda: probes.gather(x["k"], x["v"], idx, go), 20)
    t_gc = timed(lambda: probes.gather(x["k"], x["v"], idx, go), 20, cold=True)
    del idx, go
    m = 8192
    xa = torch.randn(m, m, dtype=torch.bfloat16, device="cuda:0")
    ya = torch.randn(m, m, dtype=torch.bfloat16, device="cuda:0")
    t_mm = timed(lambda: torch.matmul(xa, ya), 10)
    del xa, ya
    torch.cuda.empty_cache()
    return {"copy_GB_per_s": round(2 * 4 * n / t_copy / 1e9, 1),
            "read_stream_GB_per_s": round(8 * n / t_read / 1e9, 1),
            "row_gather_GB_per_s": round(g_bytes / t_gc / 1e9, 1),
            "row_gather_warm_GB_per_s": round(g_bytes / t_gw / 1e9, 1),
            "row_gather_note": f"probe kernel, {g_bytes} B of random K and V rows of the "
                               "decode cache (the token layer's size and pattern), cold "
                               "(after the scrub) and warm; includes its launch",
            "gemm_bf16_TFLOP_per_s": round(2 * m ** 3 / t_mm / 1e12, 1),
            "spec": {"hbm_GB_per_s": HBM_PEAK_GBS, "bf16_dense_TFLOP_per_s": BF16_PEAK_TFLOPS},
            "timing": "median"}


def block_decode_leg(args):
    """The HySparse block workload's sparse layer at its own shape in decode (batch 4, t = 65535,
    32/8 heads, d 128, bf16; 16 blocks of 64 keys + the gated 128-key window over the layer's own
    K', V': 18,874,368 B per layer), cold (after the 1 GiB read scrub) and warm, with the full attention
    and block selection that produce its index sets."""
    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, Workload, make_inputs

    w5 = WORKLOADS["block_7b_64k"]
    wl = Workload("block_7b_64k_decode", w5.batch, 1, w5.kv_len, w5.n_q_heads, w5.n_kv_heads,
                  w5.head_dim, "bf16", block=w5.block, n_blocks=w5.n_blocks, window=w5.window,
                  seed=w5.seed)
    x = make_inputs(wl, device=torch.device("cuda:0"), block_variant=True)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    swa = (x["k_loc"], x["v_loc"], x["gate"], wl.window)
    probes = Probes(torch)
    reps = max(args.steps, 10)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(reps)]

    def step(e=None):
        m = (lambda i: e[i].record()) if e else (lambda i: None)
        m(0)
        _, lse = hs.full_attn_fwd(q, k, v)
        m(1)
        bidx, bcnt = hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        m(2)
        probes.scrub()
        m(3)
        hs.sparse_attn_gather(qs, k, v, bidx, bcnt, kind="block", block=wl.block, swa=swa)
        m(4)
        hs.sparse_attn_gather(qs, k, v, bidx, bcnt, kind="block", block=wl.block, swa=swa)
        m(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for r in range(reps):
        step(ev[r])
    torch.cuda.synchronize()
    med = [sorted(e[i].elapsed_time(e[i + 1]) for e in ev)[reps // 2] for i in range(5)]
    b = costs.block_gather_bytes(wl)
    del x, q, k, v, qs, swa, probes
    torch.cuda.empty_cache()
    return {"workload": wl.name, "gathered_bytes_per_layer": b,
            "full_attn_ms": round(med[0], 4), "block_topk_ms": round(med[1], 4),
            "sparse_layer_cold_us": round(med[3] * 1e3, 2),
            "sparse_layer_cold_GB_per_s": round(rate(b, med[3]), 1),
            "sparse_layer_cold_hbm_frac": round(rate(b, med[3]) / HBM_PEAK_GBS, 3),
            "sparse_layer_warm_us": round(med[4] * 1e3, 2),
            "sparse_layer_warm_GB_per_s": round(rate(b, med[4]), 1),
            "timing": f"median of {reps}"}


def long_decode_leg(args, cpu=True):
    """The 80B shape in decode at 2^20 context (batch 4, 64/4 heads, d 128, 16 clusters of 16
    needles per KV head): full attention (K + V once: 8.59 GB), token top-k recomputed from Q and
    K, and the 11 token-sparse layers (9.44 MB gathered each); with `cpu`, the oracle's time for
    batch entry 0 (full attention + token top-k), scaled to the batch."""
    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs, to_numpy_f32

    wl = WORKLOADS["decode_80b_1m"]
    x = make_inputs(wl, device=torch.device("cuda:0"), n_sparse=1)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    reps = 5
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]

    def step(e=None):
        m = (lambda i: e[i].record()) if e else (lambda i: None)
        m(0)
        _, lse = hs.full_attn_fwd(q, k, v)
        m(1)
        idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
        m(2)
        for _ in range(wl.n_sparse):  # the layers' own Q' differ only in values
            hs.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")
        m(3)

    step()
    torch.cuda.synchronize()
    for r in range(reps):
        step(ev[r])
    torch.cuda.synchronize()
    t = [sorted(e[i].elapsed_time(e[i + 1]) for e in ev)[reps // 2] for i in range(3)]
    b_fa, b_sc, b_sp = costs.full_attn_kv_bytes(wl), costs.score_k_bytes(wl), costs.token_gather_bytes(wl)
    out = {"workload": wl.name, "ms_per_step": round(sum(t), 4), "full_attn_ms": round(t[0], 4),
           "full_attn_GB_per_s": round(b_fa / (t[0] * 1e-3) / 1e9, 1),
           "full_attn_hbm_frac": round(b_fa / (t[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
           "token_topk_ms": round(t[1], 4),
           "token_topk_GB_per_s": round(b_sc / (t[1] * 1e-3) / 1e9, 1),
           "sparse_layers_ms": round(t[2], 4),
           "sparse_per_layer_us": round(t[2] / wl.n_sparse * 1e3, 2),
           "sparse_GB_per_s": round(wl.n_sparse * b_sp / (t[2] * 1e-3) / 1e9, 1),
           "timing": "median of 5"}
    if cpu:
        import oracle
        qn, kn, vn = (to_numpy_f32(x[n][0:1]) for n in ("q", "k", "v"))
        del x, q, k, v, qs
        torch.cuda.empty_cache()
        t0 = time.perf_counter()
        _, lse = oracle.full_attention(qn, kn, vn)
        oracle.token_topk(qn, kn, lse, wl.k_global, wl.window)
        tc = time.perf_counter() - t0
        out["cpu_oracle"] = {"kind": "oracle", "cores": oracle.threads(),
                             "sample": f"batch entry 0 of {wl.batch}, full attention + token "
                                       f"top-k, {tc:.1f} s",
                             "extrapolated_s": round(tc * wl.batch, 1),
                             "gpu_s": round((t[0] + t[1]) * 1e-3, 5)}
    else:
        del x, q, k, v, qs
        torch.cuda.empty_cache()
    return out


def mqa256_leg(args):
    """HySparse2's own head shape (MQA, 64 query heads on one KV head, d 256) in decode, batch 8 at
    32k context: full attention keeping its logits, token selection from them, 3 token-sparse
    layers.  Full attention's GB/s counts K and V read once; the sparse layers' the gathered
    rows."""
    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS["decode_mqa256_32k"]
    x = make_inputs(wl, device=torch.device("cuda:0"))
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(e=None):
        m = (lambda i: e[i].record()) if e else (lambda i: None)
        m(0)
        _, lse, lg = hs.full_attn_fwd_logits(q, k, v)
        m(1)
        idx, cnt = hs.oracle_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.k_global,
                                              wl.window)
        m(2)
        for l in range(wl.n_sparse):
            hs.sparse_attn_gather(qs[l], k, v, idx, cnt, kind="token")
        m(3)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for s2 in range(args.steps):
        step(ev[s2])
    torch.cuda.synchronize()
    t = [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / args.steps for i in range(3)]
    b_fa = costs.full_attn_kv_bytes(wl)
    b_sp = costs.token_gather_bytes(wl)
    del x, q, k, v, qs
    torch.cuda.empty_cache()
    return {"workload": wl.name, "ms_per_step": round(sum(t), 4),
            "full_attn_ms": round(t[0], 4),
            "full_attn_GB_per_s": round(b_fa / (t[0] * 1e-3) / 1e9, 1),
            "full_attn_hbm_frac": round(b_fa / (t[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
            "token_select_ms": round(t[1], 4), "sparse_layers_ms": round(t[2], 4),
            "sparse_GB_per_s": round(wl.n_sparse * b_sp / (t[2] * 1e-3) / 1e9, 1)}


def block_prefill_leg(args):
    """HySparse on the 64k block workload in prefill (batch 4, 65536-query causal prefill, 32/8
    heads, d 128, bf16, blocks of 64, top 16): full attention followed by the block selection
    pass, against the one-pass call that selects inside full attention; then the gated
    block-sparse + sliding-window layer over all 65536 queries (its own Q', K', V').  TFLOP/s
    count the full-attention flops (plus the recompute flops for the two-pass version); the
    sparse layer reports its logical gathered bytes (every (b, t, u) set's 16 x 64 + 128 rows:
    1.237 TB, most of them read from cache, since neighbouring queries share blocks) and its
    4 d flops per (query head, key)."""
    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS["block_7b_64k"]
    x = make_inputs(wl, device=torch.device("cuda:0"), block_variant=True)
    q, k, v, qs = x["q"], x["k"], x["v"], x["q_sparse"][0]
    swa = (x["k_loc"], x["v_loc"], x["gate"], wl.window)
    _, lse = hs.full_attn_fwd(q, k, v)
    hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
    _, _, bidx, bcnt = hs.full_attn_block_topk(q, k, v, wl.block, wl.n_blocks)
    hs.sparse_attn_gather(qs, k, v, bidx, bcnt, kind="block", block=wl.block, swa=swa)
    torch.cuda.synchronize()
    reps = 5
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record()
        _, lse = hs.full_attn_fwd(q, k, v)
        ev[r][1].record()
        hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        ev[r][2].record()
        hs.full_attn_block_topk(q, k, v, wl.block, wl.n_blocks)
        ev[r][3].record()
        hs.sparse_attn_gather(qs, k, v, bidx, bcnt, kind="block", block=wl.block, swa=swa)
        ev[r][4].record()
    torch.cuda.synchronize()
    t_fa, t_sel, t_one, t_sp = (sum(e[i].elapsed_time(e[i + 1]) for e in ev) / reps
                                for i in range(4))
    f_fa, f_sc = costs.full_attn_flops(wl), costs.score_flops(wl)
    b_sp = costs.block_gather_bytes(wl)
    f_sp = 4 * wl.head_dim * wl.n_q_heads * (b_sp // (2 * wl.head_dim * 2 * wl.n_kv_heads))
    del x, q, k, v, qs, swa, lse, bidx, bcnt
    torch.cuda.empty_cache()
    return {"workload": wl.name, "full_attn_ms": round(t_fa, 2), "block_select_ms": round(t_sel, 2),
            "one_pass_ms": round(t_one, 2),
            "full_attn_tflops": round(f_fa / (t_fa * 1e-3) / 1e12, 1),
            "two_pass_tflops": round((f_fa + f_sc) / ((t_fa + t_sel) * 1e-3) / 1e12, 1),
            "one_pass_useful_tflops": round(f_fa / (t_one * 1e-3) / 1e12, 1),
            "speedup_one_pass": round((t_fa + t_sel) / t_one, 3),
            "sparse_layer_ms": round(t_sp, 2), "sparse_layer_logical_bytes": b_sp,
            "sparse_layer_logical_GB_per_s": round(rate(b_sp, t_sp), 1),
            "sparse_layer_tflops": round(f_sp / (t_sp * 1e-3) / 1e12, 1), "reps": reps}


def sparse_sweep(wl, batches=(8, 32, 128)):
    """The token-sparse decode layer alone (7B decode shape: 32k context, 32/8 heads, d 128,
    1024 + 128 keys per (b, u)) at several batch sizes, over synthetic sorted index sets:
    gathered K+V bytes per second against the 8 TB/s HBM peak.  At the benchmark's batch of 8
    the layer is latency-bound; larger batches show the kernel's bandwidth."""
    import torch

    from oracle_top_kv_amd import hs
    from oracle_top_kv_amd.inputs import Workload, make_inputs, random_token_sets

    res = {}
    for B in batches:
        w = Workload("sweep", B, 1, wl.kv_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16",
                     n_sparse=1, seed=600 + B)
        x = make_inputs(w, device=torch.device("cuda:0"))
        idx, cnt = random_token_sets(B, w.n_kv_heads, w.kv_len, wl.k_global, wl.window,
                                     seed=700 + B, device="cuda:0")
        qs, k, v = x["q_sparse"][0], x["k"], x["v"]
        for _ in range(3):
            hs.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for _ in range(reps):
            hs.sparse_attn_gather(qs, k, v, idx, cnt, kind="token")
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        byts = B * w.n_kv_heads * (wl.k_global + wl.window) * 2 * w.head_dim * 2
        gbs = byts / (us * 1e-6) / 1e9
        res[f"batch_{B}"] = {"us": round(us, 1), "GB_per_s": round(gbs, 1),
                             "hbm_frac": round(gbs / HBM_PEAK_GBS, 3)}
        del x, idx, cnt, qs, k, v
        torch.cuda.empty_cache()
    return res


def _host(t, b):
    return t[b:b + 1].float().cpu().numpy()


def cpu_baseline_sparse(wl, x, budget_s):
    """The oracle, as it is, running token-sparse layers (its dense masked attention over the full
    layer's index sets, which it computes first, untimed) on the host cores, batch entry after
    batch entry and layer after layer until about `budget_s` seconds have passed: gathered K+V
    bytes of the layers per second (the GPU `value`'s unit)."""
    import oracle
    from oracle_top_kv_amd import costs

    layers, t_used = 0, 0.0
    ent = {}  # per batch entry: host K, V, the sparse layers' queries and the index sets
    n_b = x["q"].shape[0]
    for it in range(64 * n_b):  # the batch entries in turn, until the budget is spent
        b = it % n_b
        if b not in ent:  # untimed
            q, k, v = _host(x["q"], b), _host(x["k"], b), _host(x["v"], b)
            _, lse = oracle.full_attention(q, k, v)
            ent[b] = (k, v, [_host(qs_l, b) for qs_l in x["q_sparse"]],
                      oracle.token_topk(q, k, lse, wl.k_global, wl.window))
        k, v, q_sp, (idx, cnt) = ent[b]
        for qs in q_sp:
            t0 = time.perf_counter()
            oracle.masked_attention(qs, k, v, idx, cnt)
            t_used += time.perf_counter() - t0
            layers += 1
        if t_used >= budget_s:
            break
    per_layer_b = costs.token_gather_bytes(wl) / wl.batch  # one batch entry's layer
    return {"value": round(layers * per_layer_b / t_used / 1e9, 4), "unit": "GB/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{layers} token-sparse layer runs over the batch entries of {wl.name} "
                      f"in turn (one entry each), {t_used:.2f} s of oracle time"}


def cpu_baseline(wl, x, budget_s):
    """The oracle, as it is, on the host cores over whole batch entries of the same workload
    (full layer, token top-k, the sparse layers, block top-k and the gated layer), the batch
    entries in turn until about `budget_s` seconds have passed; scaled to GB/s of the step's
    algorithmic bytes."""
    import oracle
    from oracle_top_kv_amd import costs

    done, t_used = 0, 0.0
    ent = {}  # host copies per batch entry (untimed)
    n_b = x["q"].shape[0]
    for it in range(16 * n_b):  # the batch entries in turn, until the budget is spent
        b = it % n_b
        if b not in ent:
            ent[b] = (_host(x["q"], b), _host(x["k"], b), _host(x["v"], b),
                      [_host(t, b) for t in x["q_sparse"]], _host(x["k_loc"], b),
                      _host(x["v_loc"], b), _host(x["gate"], b))
        q, k, v, qs, kl, vl, gate = ent[b]
        t0 = time.perf_counter()
        _, lse = oracle.full_attention(q, k, v)
        idx, cnt = oracle.token_topk(q, k, lse, wl.k_global, wl.window)
        for l in range(wl.n_sparse):
            oracle.masked_attention(qs[l], k, v, idx, cnt)
        bi, bc = oracle.block_topk(q, k, lse, wl.block, wl.n_blocks)
        oracle.gated_block_swa(qs[0], k, v, bi, bc, wl.block, kl, vl, wl.window, gate)
        t_used += time.perf_counter() - t0
        done += 1
        if t_used >= budget_s:
            break
    per_b = (costs.full_attn_kv_bytes(wl) + 2 * costs.score_k_bytes(wl) +
             wl.n_sparse * costs.token_gather_bytes(wl) + costs.block_gather_bytes(wl)) / wl.batch
    return {"value": round(done * per_b / t_used / 1e9, 4), "unit": "GB/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{done} batch-entry passes over the {wl.batch} entries of {wl.name}, "
                      f"every stage, {t_used:.1f} s of oracle time"}


def cpu_baseline_prefill(gpu_prefill, n_rows=8):
    """The oracle on a fixed sample of query rows of the 80B prefill chunk (full attention and
    token top-k for rows spread over the 4096 queries, first and last included), extrapolated by
    rows to the whole chunk and set against the GPU's time for the same two stages."""
    import numpy as np
    import torch

    import oracle
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs, to_numpy_f32

    wl = WORKLOADS["prefill_80b_128k"]
    x = make_inputs(wl, device=torch.device("cuda:0"), n_sparse=0)
    q, k, v = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    del x
    torch.cuda.empty_cache()
    rows = np.linspace(0, wl.q_len - 1, n_rows).round().astype(np.int32)
    t0 = time.perf_counter()
    _, lse = oracle.full_attention(q, k, v, rows=rows)
    oracle.token_topk(q, k, lse, wl.k_global, wl.window, rows=rows)
    t = time.perf_counter() - t0
    est = t * wl.q_len / n_rows
    out = {"kind": "oracle", "cores": oracle.threads(), "sample": f"{n_rows} of {wl.q_len} query "
           f"rows of {wl.name}, full attention + token top-k, {t:.1f} s", "extrapolated_s": round(est, 1)}
    if gpu_prefill:
        gpu_s = (gpu_prefill["full_attn_ms"] + gpu_prefill["topk_ms"]) * 1e-3
        out["gpu_s"] = round(gpu_s, 4)
        out["gpu_speedup_extrapolated"] = round(est / gpu_s, 1)
    return out


def cpu_baseline_block(gpu_block, n_rows=8):
    """The oracle on a fixed sample of query rows of the 64k block workload (full attention and
    the block top-16 for rows spread over the 65536 queries, first and last included, every
    batch entry), extrapolated by rows and set against the GPU's one-pass time for both."""
    import numpy as np
    import torch

    import oracle
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs, to_numpy_f32

    wl = WORKLOADS["block_7b_64k"]
    x = make_inputs(wl, device=torch.device("cuda:0"), n_sparse=0)
    q, k, v = (to_numpy_f32(x[n]) for n in ("q", "k", "v"))
    del x
    torch.cuda.empty_cache()
    rows = np.linspace(0, wl.q_len - 1, n_rows).round().astype(np.int32)
    t0 = time.perf_counter()
    _, lse = oracle.full_attention(q, k, v, rows=rows)
    oracle.block_topk(q, k, lse, wl.block, wl.n_blocks, rows=rows)
    t = time.perf_counter() - t0
    # the sampled rows are spread evenly over the causal range, so their mean length is the mean
    est = t * wl.q_len / n_rows
    out = {"kind": "oracle", "cores": oracle.threads(), "sample": f"{n_rows} of {wl.q_len} query "
           f"rows of {wl.name}, every batch entry, full attention + block top-{wl.n_blocks}, "
           f"{t:.1f} s", "extrapolated_s": round(est, 1)}
    if gpu_block:
        gpu_s = gpu_block["one_pass_ms"] * 1e-3
        out["gpu_s"] = round(gpu_s, 4)
        out["gpu_speedup_extrapolated"] = round(est / gpu_s, 1)
    return out


if __name__ == "__main__":
    main()
