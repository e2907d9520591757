"""Benchmark of the hot path on one MI355X.

One step = one pass of every stage of the hot path over one batch of the 7B-shaped decode
workload (batch 8, 32768-token context, 32 query / 8 KV heads, d = 128, bf16, 16 needles per KV
head):
  full attention with LSE -> token oracle top-k (1024 + window 128) -> 3 token-sparse layers
  (each with its own Q') -> block scores + top-16 blocks -> a block-sparse layer with its gated
  sliding-window branch (own K', V').
Inputs are generated on the GPU before timing and stay resident in HBM.

Prints ONE JSON line.  `value` is the step's algorithmic HBM bytes (what the method must read: K
and V once for full attention, K once for each scoring pass, the index-set rows of K and V for
each sparse layer) divided by the step time (`ms_per_step_graph`: the same step replayed from a
HIP graph).  `step_stored_logits` times the same step with full attention keeping its logits
and both selections reading them back instead of re-reading K (its own bytes and GB/s).
Per-stage times come from HIP events recorded on the stream the library launches on.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_7b_32k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 80B-shaped prefill leg (full attention + token top-k)")
    ap.add_argument("--no-block-prefill", action="store_true",
                    help="skip the 64k block-selection prefill leg (HySparse scoring pass)")
    ap.add_argument("--no-long-decode", action="store_true",
                    help="skip the 2^20-context decode leg (80B shape)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the token-sparse decode layer sweep over batch sizes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (calibrates the "
                         "HBM byte counters of a profiler) and exit")
    return ap.parse_args()


def copy_probe(mib):
    """A plain copy kernel of known size: reads and writes exactly `mib` MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 5}), flush=True)


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
    torch.cuda.synchronize()

    stages = ["full_attn", "token_topk", "sparse_token", "block_topk", "sparse_block_swa"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        o, lse = hs.full_attn_fwd(q, k, v)
        mark(1)
        idx, cnt = hs.oracle_topk(q, k, lse, wl.k_global, wl.window)
        mark(2)
        for l in range(wl.n_sparse):
            hs.sparse_attn_gather(qs[l], k, v, idx, cnt, kind="token")
        mark(3)
        bidx, bcnt = hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        mark(4)
        hs.sparse_attn_gather(qs[0], k, v, bidx, bcnt, kind="block", block=wl.block,
                              swa=(kl, vl, gate, wl.window))
        mark(5)

    # The same step with the selection reading the logits that full attention stored, instead
    # of recomputing them from Q and K (decode only: the logits are B * Hq * kv_len floats).
    def step_logits(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        o, lse, lg = hs.full_attn_fwd_logits(q, k, v)
        mark(1)
        idx, cnt = hs.oracle_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.k_global,
                                              wl.window)
        mark(2)
        for l in range(wl.n_sparse):
            hs.sparse_attn_gather(qs[l], k, v, idx, cnt, kind="token")
        mark(3)
        bidx, bcnt = hs.block_topk_from_logits(lg, lse, wl.n_kv_heads, wl.head_dim, wl.block,
                                               wl.n_blocks)
        mark(4)
        hs.sparse_attn_gather(qs[0], k, v, bidx, bcnt, kind="block", block=wl.block,
                              swa=(kl, vl, gate, wl.window))
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, bracketed by synchronization, with per-stage events
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step(evs[s])
    t_end.record()
    torch.cuda.synchronize()
    ms_step_eager = t_start.elapsed_time(t_end) / args.steps
    stage_ms = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                for i, name in enumerate(stages)}
    stage_all = {name: sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
                 for i, name in enumerate(stages)}

    # The same step captured once in a HIP graph and replayed (reported as ms_per_step_graph):
    # the library allocates nothing, never synchronizes and zero-fills with kernels, so every
    # call is capturable.  Measured equal to the eager step: launches already run ahead of the
    # GPU, so there are no host gaps to remove.
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    g_start = torch.cuda.Event(enable_timing=True)
    g_end = torch.cuda.Event(enable_timing=True)
    g_start.record()
    for _ in range(args.steps):
        graph.replay()
    g_end.record()
    torch.cuda.synchronize()
    ms_step_graph = g_start.elapsed_time(g_end) / args.steps
    del graph
    ms_step = ms_step_eager

    # the stored-logits step, timed the same way (eager)
    for _ in range(args.warmup):
        step_logits()
    evl = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step_logits(evl[s])
    t_end.record()
    torch.cuda.synchronize()
    ms_step_logits = t_start.elapsed_time(t_end) / args.steps
    stage_ms_logits = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evl) / args.steps
                       for i, name in enumerate(stages)}

    # algorithmic bytes per stage
    b_full = costs.full_attn_kv_bytes(wl)                 # K and V read once
    b_score = costs.score_k_bytes(wl)                     # K read once per scoring pass
    b_tok = costs.token_gather_bytes(wl)                  # per sparse layer
    b_blk = costs.block_gather_bytes(wl)                  # per block-sparse + SWA layer
    stage_bytes = {"full_attn": b_full, "token_topk": b_score,
                   "sparse_token": wl.n_sparse * b_tok, "block_topk": b_score,
                   "sparse_block_swa": b_blk}
    total_bytes = sum(stage_bytes.values())
    value = total_bytes / (ms_step * 1e-3) / 1e9

    stages_out = {}
    for n in stages:
        gbs = stage_bytes[n] / (stage_ms[n] * 1e-3) / 1e9
        v = stage_all[n]
        stages_out[n] = {"ms": round(stage_ms[n], 4), "median_ms": round(v[len(v) // 2], 4),
                         "min_ms": round(v[0], 4), "GB_per_s": round(gbs, 1),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 3)}
    stages_out["sparse_token"]["per_layer_gathered_bytes"] = b_tok
    dom = "full_attn"
    achieved = stage_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9

    # stored-logits step: full attention also writes the logits; each selection reads them back
    b_logits = costs.logit_bytes(wl)
    stage_bytes_l = {"full_attn": b_full + b_logits, "token_topk": b_logits,
                     "sparse_token": wl.n_sparse * b_tok, "block_topk": b_logits,
                     "sparse_block_swa": b_blk}
    total_bytes_l = sum(stage_bytes_l.values())
    logits_out = {"ms_per_step": round(ms_step_logits, 4), "step_bytes": total_bytes_l,
                  "GB_per_s": round(total_bytes_l / (ms_step_logits * 1e-3) / 1e9, 1),
                  "speedup_vs_recompute": round(ms_step / ms_step_logits, 3), "stages": {}}
    for n in stages:
        gbs = stage_bytes_l[n] / (stage_ms_logits[n] * 1e-3) / 1e9
        logits_out["stages"][n] = {"ms": round(stage_ms_logits[n], 4), "GB_per_s": round(gbs, 1),
                                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 3)}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_graph": round(ms_step_graph, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "kv_len": wl.kv_len,
                   "q_len": wl.q_len, "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "k_global": wl.k_global, "window": wl.window,
                   "sparse_layers": wl.n_sparse, "block": wl.block, "n_blocks": wl.n_blocks,
                   "needles_per_kv_head": wl.needles, "step_bytes": total_bytes},
        "stages": stages_out,
        "roofline": {"bound": "hbm",
                     "kernel": "full-attention decode call (row_attn_kernel + combine_kernel)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": b_full, "traffic": counter_traffic(wl.name)},
        "step_stored_logits": logits_out,
    }
    out["step_paged"] = paged_step(wl, x, hs, args, logits_out["ms_per_step"])
    out["sparse_cold_cache"] = cold_sparse(wl, x, hs, costs)
    peaks = measured_peaks()
    out["measured_peaks"] = peaks
    out["roofline"]["frac_of_measured_copy"] = round(achieved / peaks["copy_GB_per_s"], 4)
    if not args.no_prefill or not args.no_sweep:
        del x, q, k, v, qs, kl, vl, gate
        torch.cuda.empty_cache()
    gemm = peaks["gemm_bf16_TFLOP_per_s"]
    if not args.no_prefill:
        out["prefill"] = prefill_leg(args)
        out["prefill"]["full_attn_frac_of_measured_gemm"] = round(
            out["prefill"]["full_attn_tflops"] / gemm, 4)
    if not args.no_block_prefill:
        out["block_prefill"] = block_prefill_leg(args)
    out["mqa256_decode"] = mqa256_leg(args)
    if not args.no_long_decode:
        out["long_decode"] = long_decode_leg(args, cpu=not args.no_cpu_baseline)
    if not args.no_sweep:
        out["sparse_decode_sweep"] = sparse_sweep(wl)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, make_inputs(wl, device=dev, block_variant=True),
                                           args.cpu_seconds)
        if not args.no_prefill:
            out["cpu_baseline_prefill"] = cpu_baseline_prefill(out.get("prefill"))
        if not args.no_block_prefill:
            out["cpu_baseline_block"] = cpu_baseline_block(out.get("block_prefill"))
    print(json.dumps(out), flush=True)


def counter_traffic(workload):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading); None when that summary
    is missing, covers another workload, or any kernel source it lists has changed since."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    meta = json.loads(m.group(1))
    if meta.get("workload") != workload:
        return None
    for rel, digest in meta["sources_sha256"].items():
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != digest:
            return None
    return meta["traffic_bytes_per_launch"]


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
    reps = 3
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
    f_fa, f_sc = costs.full_attn_flops(wl), costs.score_flops(wl)
    tot = (f_fa + f_sc) / ((t_fa + t_tk) * 1e-3) / 1e12
    b_sp = costs.token_gather_bytes(wl)  # rows each (b, t, u) gathers (mostly from cache)
    f_sp = costs.sparse_flops(wl)
    return {"workload": wl.name, "full_attn_ms": round(t_fa, 3), "topk_ms": round(t_tk, 3),
            "full_attn_tflops": round(f_fa / (t_fa * 1e-3) / 1e12, 1),
            "topk_score_tflops": round(f_sc / (t_tk * 1e-3) / 1e12, 1),
            "full_attn_plus_topk_tflops": round(tot, 1),
            "useful_tflops": round(f_fa / ((t_fa + t_tk) * 1e-3) / 1e12, 1),
            "mfma_frac_full_attn": round(f_fa / (t_fa * 1e-3) / 2.5e15, 4),
            "sparse_layer_ms": round(t_sp, 3),
            "sparse_layer_logical_GB_per_s": round(b_sp / (t_sp * 1e-3) / 1e9, 1),
            "sparse_layer_tflops": round(f_sp / (t_sp * 1e-3) / 1e12, 1),
            "peak_tflops": 2500.0, "reps": reps}


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


def cold_sparse(wl, x, hs, costs, reps=10):
    """One token-sparse layer and the gated block layer, each timed alone right after a 1 GiB
    scrub write, so that neither the 256 MB last-level cache nor L2 holds the gathered rows (the
    step's own numbers are warm: the layers run back to back after full attention)."""
    import torch

    scrub = torch.empty(1 << 28, dtype=torch.float32, device=x["q"].device)
    _, lse = hs.full_attn_fwd(x["q"], x["k"], x["v"])
    idx, cnt = hs.oracle_topk(x["q"], x["k"], lse, wl.k_global, wl.window)
    bidx, bcnt = hs.block_score_topk(x["q"], x["k"], lse, wl.block, wl.n_blocks)
    calls = {
        "sparse_token": (lambda: hs.sparse_attn_gather(x["q_sparse"][0], x["k"], x["v"], idx, cnt,
                                                       kind="token"),
                         costs.token_gather_bytes(wl)),
        "sparse_block_swa": (lambda: hs.sparse_attn_gather(
            x["q_sparse"][0], x["k"], x["v"], bidx, bcnt, kind="block", block=wl.block,
            swa=(x["k_loc"], x["v_loc"], x["gate"], wl.window)), costs.block_gather_bytes(wl)),
    }
    res = {}
    for name, (fn, byts) in calls.items():
        fn()
        ts = []
        for r in range(reps):
            scrub.fill_(float(r))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        med = ts[len(ts) // 2]
        res[name] = {"median_us": round(med, 1), "min_us": round(ts[0], 1),
                     "GB_per_s": round(byts / (med * 1e-6) / 1e9, 1),
                     "hbm_frac": round(byts / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                     "bytes": byts, "reps": reps}
    del scrub
    return res


def measured_peaks():
    """Peaks measured on this GPU with library kernels: a 1 GiB device copy (bytes read plus
    written per second) and a large bf16 GEMM (dense MFMA, TFLOP/s)."""
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    t_copy = timed(lambda: b.copy_(a), 10)
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device="cuda:0")
    y = torch.randn(m, m, dtype=torch.bfloat16, device="cuda:0")
    t_mm = timed(lambda: torch.matmul(x, y), 10)
    del x, y
    torch.cuda.empty_cache()
    return {"copy_GB_per_s": round(2 * 4 * n / t_copy / 1e9, 1),
            "gemm_bf16_TFLOP_per_s": round(2 * m ** 3 / t_mm / 1e12, 1),
            "spec": {"hbm_GB_per_s": HBM_PEAK_GBS, "bf16_dense_TFLOP_per_s": 2500.0}}


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
    """HySparse scoring on the 64k block workload (batch 4, 65536-query causal prefill, 32/8
    heads, d 128, bf16, blocks of 64, top 16): full attention followed by the block selection
    pass, against the one-pass call that selects inside full attention.  TFLOP/s count the
    full-attention flops (plus the recompute flops for the two-pass version)."""
    import torch

    from oracle_top_kv_amd import costs, hs
    from oracle_top_kv_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS["block_7b_64k"]
    x = make_inputs(wl, device=torch.device("cuda:0"), n_sparse=0)
    q, k, v = x["q"], x["k"], x["v"]
    _, lse = hs.full_attn_fwd(q, k, v)
    hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
    hs.full_attn_block_topk(q, k, v, wl.block, wl.n_blocks)
    torch.cuda.synchronize()
    reps = 2
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record()
        _, lse = hs.full_attn_fwd(q, k, v)
        ev[r][1].record()
        hs.block_score_topk(q, k, lse, wl.block, wl.n_blocks)
        ev[r][2].record()
        hs.full_attn_block_topk(q, k, v, wl.block, wl.n_blocks)
        ev[r][3].record()
    torch.cuda.synchronize()
    t_fa = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    t_sel = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    t_one = sum(e[2].elapsed_time(e[3]) for e in ev) / reps
    f_fa, f_sc = costs.full_attn_flops(wl), costs.score_flops(wl)
    del x, q, k, v, lse
    torch.cuda.empty_cache()
    return {"workload": wl.name, "full_attn_ms": round(t_fa, 2), "block_select_ms": round(t_sel, 2),
            "one_pass_ms": round(t_one, 2),
            "two_pass_tflops": round((f_fa + f_sc) / ((t_fa + t_sel) * 1e-3) / 1e12, 1),
            "one_pass_useful_tflops": round(f_fa / (t_one * 1e-3) / 1e12, 1),
            "speedup_one_pass": round((t_fa + t_sel) / t_one, 3), "reps": reps}


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


def cpu_baseline(wl, x, budget_s):
    """The oracle, as it is, on the host cores over whole batch entries of the same workload
    (full layer, token top-k, the sparse layers, block top-k and the gated layer), taken one batch
    entry at a time until about `budget_s` seconds have passed; scaled to GB/s of the same
    algorithmic bytes."""
    import numpy as np

    import oracle
    from oracle_top_kv_amd import costs

    def host(t, b):
        return t[b:b + 1].float().cpu().numpy()

    done, t_used = 0, 0.0
    for b in range(wl.batch):
        q, k, v = host(x["q"], b), host(x["k"], b), host(x["v"], b)
        qs = [host(t, b) for t in x["q_sparse"]]
        kl, vl, gate = host(x["k_loc"], b), host(x["v_loc"], b), host(x["gate"], b)
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
            "sample": f"{done} of {wl.batch} batch entries, every stage, {t_used:.1f} s"}


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
