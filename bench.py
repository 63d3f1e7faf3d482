"""Benchmark: drift-refresh steps/s of the 32-layer LLaDA-8B-shaped stack on one MI355X.

A step is one refresh step through every layer (window update, QKV projection
with K/V patching, attention + proxy-attention KL drift + top-k, gathered
sparse forward producing the update packet), plus the last layer's
main-attention drift for the commit rule, on synthetic bf16 data:
hidden 4096, 32 heads x 128, FFN 12288 SwiGLU, prompt 512 + gen 512, B = 32,
window 96 (2B prefix + B suffix), K = 8 clusters, top-k = 4.  Inputs are
resident in HBM before the timed region; the whole step is one HIP graph.

Prints one JSON line.  --gpus N with N > 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD specification
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD specification
METRIC = "drift-refresh steps/s (32-layer LLaDA-8B shape) + % peak HBM GB/s, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(w, n_sel: float) -> dict:
    """Algorithmic HBM bytes of one refresh step of one layer (weights once, KV once, state r/w)."""
    d, hq, hkv, dh, F, n, Bk = w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn, w.n_pos, w.block
    nq, nkv = hq * dh, hkv * dh
    nw = w.win_prefix + w.win_suffix
    rows = Bk + n_sel
    b = {
        "w_qkv": 2 * d * (nq + 2 * nkv), "w_o": 2 * nq * d, "w_gu": 2 * 2 * F * d, "w_down": 2 * F * d,
        "kv_read": 2 * 2 * n * nkv,
        "kv_write": 2 * 2 * (Bk + n_sel) * nkv,
        "proxy_logits": 2 * 4 * w.n_clusters * hq * n,
        "window": 2 * 2 * nw * d + 2 * w.n_clusters * d * 2,
        "packet": 2 * 2 * n_sel * d + 2 * 2 * Bk * d,
    }
    b["gu_launch"] = b["w_gu"] + rows * d * 4 + rows * F * 4
    return b


def counter_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None when the projection sources changed since the counters were taken."""
    import re
    from drift_driven_sparse_amd import prof_summary
    path = os.path.join(ROOT, "profiles", "gate_up_projection_llada8b_pmc.md")
    try:
        text = open(path).read()
        m = re.search(r"```json\n(.*?)\n```", text, re.S)
        rec = json.loads(m.group(1))
    except (OSError, AttributeError, ValueError):
        return None
    return rec["traffic_bytes"] if rec.get("source_hash") == prof_summary.source_hash() else None


def cpu_baseline(w, budget_s: float = 12.0):
    """The CPU oracle on a bounded sample of the same workload: whole refresh steps of
    single layers (fp64 NumPy/BLAS), weights already in host memory, timed per layer."""
    import numpy as np
    import torch

    import synth
    from oracle import polestar_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    cfg = O.Cfg.from_workload(w)
    dev = "cuda" if torch.cuda.is_available() else "cpu"
    blk = w.prompt
    wpos = O.window_positions(blk, w.n_pos, w.block, w.win_prefix, w.win_suffix)
    nw = len(wpos)
    t_total, layers = 0.0, 0
    for l in range(w.n_layers):
        W = {k: v.double().cpu().numpy() for k, v in synth.layer_weights(w, l, device=dev).items()}
        t = lambda tag, shape, dtype="bf16": synth.tensor(w, (l,) + tag, shape, 1.0, 0, dev, dtype).double().cpu().numpy()
        H = t((1,), (nw, w.d))
        ls = {"K": t((2,), (w.n_pos, w.n_kv_heads, w.head_dim)), "V": t((3,), (w.n_pos, w.n_kv_heads, w.head_dim)),
              "P": t((4,), (w.n_clusters, w.n_heads, w.n_pos), "f32")}
        z, m, _ = O.spherical_kmeans(H, w.n_clusters, synth.kmeans_init(w, nw, l, 0), w.kmeans_iters)
        ls.update(Z=cfg.st(z), M=m, H=H)
        h_act = t((5,), (w.block, w.d))
        t0 = time.perf_counter()
        cu = O.cluster_update(ls, cfg)
        dr = O.drift_layer(ls, W, cfg, blk, h_act, cu["h"], cu["patched"], True)
        O.refresh_layer(W, cfg, h_act, cu["h"], dr["o"], dr["S"])
        t_total += time.perf_counter() - t0
        layers += 1
        del W
        if t_total >= budget_s:
            break
    per_layer = t_total / layers
    return {"value": 1.0 / (per_layer * w.n_layers), "unit": "refresh-steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{layers} of {w.n_layers} layers of one refresh step (window update, drift, sparse "
                      f"forward), {t_total:.1f} s of CPU time, scaled to a {w.n_layers}-layer step"}


def entry_cpu_baseline(w, blk: int, full: bool, budget_s: float = 20.0):
    """The CPU oracle's block entry on a bounded sample: single layers of the whole-stack entry
    (forward of the entry rows over the cache, k-means, codes, proxy logits; fp64), scaled to
    the stack."""
    import numpy as np
    import torch

    import synth
    from oracle import polestar_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    cfg = O.Cfg.from_workload(w)
    dev = "cuda" if torch.cuda.is_available() else "cpu"
    rows = O.entry_positions(blk, w.n_pos, w.block, w.win_prefix, w.win_suffix, full)
    nw = len(O.window_positions(blk, w.n_pos, w.block, w.win_prefix, w.win_suffix))
    h = synth.embeddings(w, 0, dev).to(torch.bfloat16).double().cpu().numpy()
    t_total, layers = 0.0, 0
    for l in range(w.n_layers):
        W = {k: v.double().cpu().numpy() for k, v in synth.layer_weights(w, l, device=dev).items()}
        K = synth.tensor(w, (l, 10), (w.n_pos, w.n_kv_heads, w.head_dim), 1.0, 0, dev, "bf16").double().cpu().numpy()
        V = synth.tensor(w, (l, 11), (w.n_pos, w.n_kv_heads, w.head_dim), 1.0, 0, dev, "bf16").double().cpu().numpy()
        t0 = time.perf_counter()
        out = O.layer_forward_rows(h[rows], rows, W, cfg, K, V)
        O.block_entry_layer_state(h, K, V, W["wq"], cfg, blk, synth.kmeans_init(w, nw, l, 0))
        t_total += time.perf_counter() - t0
        layers += 1
        h = h.copy()
        h[rows] = out
        del W
        if t_total >= budget_s:
            break
    ms = t_total / layers * w.n_layers * 1e3
    return {"value": round(ms, 1), "unit": "ms per block entry", "cores": int(threads), "kind": "oracle",
            "sample": f"{layers} of {w.n_layers} layers of the {'full' if full else 'window'} entry, "
                      f"{t_total:.1f} s of CPU time, scaled to {w.n_layers} layers"}


def entry_flops(w, rows: int, n_layers: int) -> float:
    """Algorithmic flops of the block-entry forward of `rows` rows: the four projections and the
    two attention products over all n_pos keys."""
    nq, nkv = w.n_heads * w.head_dim, w.n_kv_heads * w.head_dim
    proj = 2.0 * rows * (w.d * (nq + 2 * nkv) + nq * w.d + 2 * w.d * w.ffn + w.ffn * w.d)
    attn = 4.0 * rows * w.n_pos * nq
    return n_layers * (proj + attn)


def entry_timing(st, w, blk, h0, inits, n_layers, reps=3):
    import torch
    from drift_driven_sparse_amd import binding as B
    res = {}
    for name, full in (("full", True), ("window", False)):
        # captured in a HIP graph like the step (the k-means is a chain of short launches); replays
        # are timed
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            st.entry_forward(blk, h0, inits, full=full)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.entry_forward(blk, h0, inits, full=full)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / reps
        del g
        rows = w.n_pos if full else min(w.n_pos, blk + w.block + w.win_suffix) - max(0, blk - w.win_prefix)
        tf = entry_flops(w, rows, n_layers) / (ms * 1e-3) / 1e12
        # one more run with HIP events around every launch (summed per kernel kind)
        B.polestar_profile(st.h, True)
        st.entry_forward(blk, h0, inits, full=full)
        prof = B.polestar_profile_read(st.h)
        B.polestar_profile(st.h, False)
        kern = {k: round(v[0], 3) for k, v in prof.items() if v[1]}
        res[name] = {"ms": round(ms, 3), "rows": rows, "TFLOPs": round(tf, 1),
                     "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "kernel_ms": kern}
        log(f"[bench] block entry ({name}, {rows} rows x {n_layers} layers): {ms:.2f} ms, {tf:.1f} TFLOP/s; "
            f"per kind (ms, eager, events around each launch): {kern}")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true", help="launch every kernel from the host loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=None, help="(diagnostics) fewer layers than the workload")
    ap.add_argument("--entry", action="store_true",
                    help="time the block entry (polestar_entry, full and window kinds) instead of the step")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="also run one element-wise copy of MB MiB (reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this refresh path runs on a single MI355X and uses no "
              "collectives; run it without --gpus or with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only (WORLD_SIZE > 1 refused).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from drift_driven_sparse_amd import binding as B
    from drift_driven_sparse_amd.stack import RefreshStack

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    w = synth.WORKLOADS[3]
    n_layers = args.layers or w.n_layers
    dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn, n_pos=w.n_pos,
                  batch=1, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix,
                  n_clusters=w.n_clusters, top_k=w.top_k, vocab=0, dtype=B.BF16, resid_fmt=B.RESID_RAW)
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist, mask_id=0,
                      kmeans_iters=w.kmeans_iters)
    t0 = time.time()
    st = RefreshStack(dims, params, n_layers)
    blk = w.prompt
    nw = st.win_max
    entry_rows, inits = [], []
    for l in range(n_layers):
        st.set_layer_weights(l, synth.layer_weights(w, l, device="cuda"))
        L = st.layers[l]
        L["k_cache"].copy_(synth.tensor(w, (l, 10), L["k_cache"].shape, 1.0, 0, "cuda", "bf16"))
        L["v_cache"].copy_(synth.tensor(w, (l, 11), L["v_cache"].shape, 1.0, 0, "cuda", "bf16"))
        L["win_h"].copy_(synth.tensor(w, (l, 12), L["win_h"].shape, 1.0, 0, "cuda", "bf16"))
        entry_rows.append(L["win_h"])
        inits.append(torch.tensor(synth.kmeans_init(w, nw, l, 0), dtype=torch.int32, device="cuda")[None])
    torch.cuda.synchronize()
    log(f"[bench] weights and state of {n_layers} layers ready in {time.time() - t0:.1f}s")
    if args.entry:
        # block entry of the whole stack from seeded layer-0 rows of every position
        h0 = synth.embeddings(w, 0, "cuda").to(torch.bfloat16)[None].contiguous()
        res = entry_timing(st, w, blk, h0, inits, n_layers)
        st.close()
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle's block entry on a bounded sample")
            for name, full in (("full", True), ("window", False)):
                res[name]["cpu_baseline"] = entry_cpu_baseline(w, blk, full, budget_s=10.0)
        print(json.dumps({"metric": "block entry ms (32-layer LLaDA-8B shape), 1 GPU", "unit": "ms",
                          "higher_is_better": False, "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": f"{w.name}: {n_layers} layers, n {w.n_pos}, block start {blk}",
                                     "layers": n_layers}, "block_entry": res}), flush=True)
        return
    # clustering of seeded window rows: the state a block entry leaves (the dense forward that
    # produces it is timed with --entry)
    st.block_entry(blk, entry_rows, inits)
    n_in = args.warmup + args.steps + 1
    inputs = synth.tensor(w, (99,), (n_in, 1, w.block, w.d), 1.0, 0, "cuda", "bf16")
    h_in = torch.zeros(1, w.block, w.d, dtype=torch.bfloat16, device="cuda")
    # first refresh step establishes the drift references (proxy and active logits)
    h_in.copy_(inputs[0])
    st.step(blk, h_in)
    torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            st.step(blk, h_in)          # eager run on the capture stream (lazy init)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            st.step(blk, h_in)
        torch.cuda.synchronize()
        log("[bench] step captured in a HIP graph")

    def run_step(i, eager=False):
        h_in.copy_(inputs[i])
        if graph is not None and not eager:
            graph.replay()
        else:
            st.step(blk, h_in)

    def timed(first, eager):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            run_step(first + i, eager)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1)

    for i in range(args.warmup):
        run_step(1 + i)
    torch.cuda.synchronize()
    if graph is None:
        B.polestar_profile(st.h, True)
    ms_total = timed(1 + args.warmup, graph is None)
    ms_step = ms_total / args.steps
    log(f"[bench] {args.steps} steps in {ms_total:.2f} ms ({ms_step:.3f} ms/step, graph={graph is not None})")
    # per-kernel durations: HIP events around every launch of an eager pass (events recorded
    # inside a captured graph carry no timestamps on this runtime).  A GPU spin queued first
    # keeps the GPU busy while the host queues the profiled steps, so the GPU runs them back to
    # back and each event interval holds the kernel's own time, not host launch gaps.
    eager_ms_step = None
    if graph is not None:
        prof_steps = 3
        probe0, probe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        probe0.record()
        torch.cuda._sleep(1_000_000)
        probe1.record()
        torch.cuda.synchronize()
        spin_cycles = int(1_000_000 * 80.0 / max(probe0.elapsed_time(probe1), 1e-3))   # about 80 ms
        B.polestar_profile(st.h, True)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(spin_cycles)
        ev0.record()
        for i in range(prof_steps):
            run_step(1 + args.warmup + i, True)
        ev1.record()
        torch.cuda.synchronize()
        eager_ms_step = ev0.elapsed_time(ev1) / prof_steps
        log(f"[bench] profiled eager pass (queued behind a GPU spin): {eager_ms_step:.3f} ms/step")
    prof = B.polestar_profile_read(st.h)
    B.polestar_profile(st.h, False)

    # selected-row counts per layer (instrumented eager step, outside the timed region)
    counts = []
    h_in.copy_(inputs[-1])
    cur = 0
    st.h_act[0].copy_(h_in)
    u_in = None
    for l in range(n_layers):
        Ls = st.struct(l)
        B.polestar_cluster(st.h, B.CLUSTER_UPDATE, Ls, blk, u_in, None, None, None, st.ws, st.ws_bytes)
        sel = st.packets[l % 2]
        B.polestar_drift(st.h, B.DRIFT_REFRESH, Ls, blk, st.h_act[cur], u_in, st.D, st.topk, sel, None, None, st.ws,
                         st.ws_bytes)
        B.polestar_refresh(st.h, Ls, blk, st.h_act[cur], sel, None, None, None, st.h_act[1 - cur], st.pk_rows[l % 2],
                           st.ws, st.ws_bytes)
        counts.append(int(st.pk_cnt[l % 2][0]))
        u_in, cur = sel, 1 - cur
    n_sel = sum(counts) / len(counts)

    lb = layer_bytes(w, n_sel)
    step_bytes = n_layers * sum(v for k, v in lb.items() if k != "gu_launch") + 2 * 2 * 4 * w.block * w.n_heads * w.n_pos
    per = {k: (v[0] / max(v[1], 1), v[1]) for k, v in prof.items() if v[1]}
    gu_ms, gu_n = per.get("gu", (float("nan"), 0))
    achieved = lb["gu_launch"] / (gu_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": "gate/up projection (split-K bf16 GEMM + SwiGLU finish)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic(),
            "bytes_per_launch": lb["gu_launch"], "avg_launch_ms": round(gu_ms, 5), "launches": gu_n,
            "timing": "HIP events around each launch of the kernel in an eager pass of the same step, "
                      "queued behind a GPU spin so that the launches run back to back"}
    kern = {k: {"avg_ms": round(v[0], 5), "launches": v[1]} for k, v in per.items()}
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(1000.0 / ms_step, 3), "unit": "refresh-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {n_layers} layers, hidden {w.d}, {w.n_heads}x{w.head_dim} heads, "
                               f"FFN {w.ffn}, prompt {w.prompt} + gen {w.gen}, B {w.block}, window "
                               f"{w.win_prefix}+{w.win_suffix}, K {w.n_clusters}, top-k {w.top_k}",
                   "layers": n_layers, "n_pos": w.n_pos, "graph": graph is not None,
                   "profiled_eager_ms_per_step": None if eager_ms_step is None else round(eager_ms_step, 4),
                   "mean_selected_rows": round(n_sel, 2)},
        "step_hbm": {"algorithmic_bytes": int(step_bytes), "achieved_GBs": round(step_gbs, 1),
                     "frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "kernels": kern,
    }
    if args.copy_probe > 0:
        src = torch.ones(args.copy_probe * (1 << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: one element-wise kernel reading {src.numel() * 4} B and writing "
            f"{dst.numel() * 4} B")
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    st.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
