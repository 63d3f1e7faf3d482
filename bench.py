"""Benchmark: drift-refresh steps/s of the 32-layer LLaDA-8B-shaped stack on one MI355X.

A step is one refresh step through every layer (window update, QKV projection
with K/V patching, attention + proxy-attention KL drift + top-k, gathered
sparse forward producing the update packet), plus the last layer's
main-attention drift for the commit rule, on synthetic bf16 data:
hidden 4096, 32 heads x 128, FFN 12288 SwiGLU, prompt 512 + gen 512, B = 32,
window 96 (2B prefix + B suffix), K = 8 clusters, top-k = 4.  Inputs are
resident in HBM before the timed region; the whole step is one HIP graph.

--workload selects another stack: the 28-layer Dream-7B-shaped GQA stack
(28 / 4 heads, FFN 18944, prompt 384 + gen 256), or 16 LLaDA-shaped sequences
of prompt 512 + gen 256 with NVFP4 window residuals whose step ends with the
commit (LM head over 126464 ids, drift spike, thresholds).

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


def window_row_bytes(w) -> int:
    """Bytes of one stored window row: raw bf16, or residual codes and scales."""
    d = w.d
    return {"raw": 2 * d, "nvfp4": d // 2 + d // 16, "fp8": d, "mxint8": d + d // 32, "mxfp4": d // 2 + d // 32}[w.resid]


def layer_bytes(w, n_sel: float, batch: int = 1) -> dict:
    """Algorithmic HBM bytes of one refresh step of one layer for `batch` sequences: every weight
    once; per sequence the K and V of all n keys once, the K/V rows written, the previous proxy
    logits read and written, the window state read and written and the packet and active rows."""
    d, hq, hkv, dh, F, n, Bk = w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn, w.n_pos, w.block
    nq, nkv = hq * dh, hkv * dh
    nw = w.win_prefix + w.win_suffix
    rows = Bk + n_sel
    b = {
        "w_qkv": 2 * d * (nq + 2 * nkv), "w_o": 2 * nq * d, "w_gu": 2 * 2 * F * d, "w_down": 2 * F * d,
        "kv_read": batch * 2 * 2 * n * nkv,
        "kv_write": batch * 2 * 2 * (Bk + n_sel) * nkv,
        "proxy_logits": batch * 2 * 4 * w.n_clusters * hq * n,
        "window": batch * (2 * nw * window_row_bytes(w) + 2 * w.n_clusters * d * 2),
        "packet": batch * (2 * 2 * n_sel * d + 2 * 2 * Bk * d),
    }
    b["gu_launch"] = b["w_gu"] + batch * (rows * d * 4 + rows * F * 4)
    return b


def layer_flops(w, n_sel: float, n_patch: float, batch: int = 1) -> dict:
    """Algorithmic flops of one refresh step of one layer for `batch` sequences, counting only the
    rows the method needs: Q/K/V of the active rows, K/V of the patched window rows, Q of the
    selected rows and of the centroids, attention of the active and selected rows over all keys
    (logits and outputs) and the centroids' logits, and the O, gate/up and down projections of
    the active and selected rows."""
    d, hq, hkv, dh, F, n, Bk, K = w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn, w.n_pos, w.block, w.n_clusters
    nq, nkv = hq * dh, hkv * dh
    tok = Bk + n_sel
    f = {
        "qkv": 2 * d * ((nq + 2 * nkv) * Bk + 2 * nkv * n_patch + nq * (n_sel + K)),
        "attn": 4 * n * nq * tok + 2 * n * nq * K,
        "o": 2 * nq * d * tok, "gu": 2 * d * 2 * F * tok, "down": 2 * F * d * tok,
    }
    return {k: v * batch for k, v in f.items()}


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


def host_info() -> dict:
    """CPU model (name, family/model/stepping, clock) and the BLAS thread count the oracle runs with."""
    model = "unknown"
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k in ("model name", "cpu family", "model", "stepping", "cpu MHz", "cache size") and k not in fields:
                fields[k] = v
            if not line.strip() and fields:
                break
        if "model name" in fields:
            model = (f"{fields['model name']} (family {fields.get('cpu family', '?')}, model "
                     f"{fields.get('model', '?')}, stepping {fields.get('stepping', '?')}, "
                     f"{fields.get('cpu MHz', '?')} MHz, cache {fields.get('cache size', '?')})")
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    return {"cpu_model": model, "blas_threads": int(threads), "host_cpus": os.cpu_count()}


def cpu_baseline(w, budget_s: float = 12.0, passes: int = 3):
    """The CPU oracle on a bounded sample of the same workload: whole refresh steps of single
    layers of one sequence (window update, drift, sparse forward; fp64 NumPy/BLAS), each layer
    run ``passes`` times with its weights already in host memory, timed per layer pass and
    scaled to the stack and the batch; with a vocabulary, also the last layer's commit (LM-head
    confidence and decision) once."""
    import numpy as np
    import torch

    import synth
    from oracle import polestar_oracle as O
    info = host_info()
    cfg = O.Cfg.from_workload(w)
    dev = "cuda" if torch.cuda.is_available() else "cpu"
    blk = w.prompt
    wpos = O.window_positions(blk, w.n_pos, w.block, w.win_prefix, w.win_suffix)
    nw = len(wpos)
    t_total, layers = 0.0, 0
    h_act = None
    for l in range(w.n_layers):
        W = {k: v.double().cpu().numpy() for k, v in synth.layer_weights(w, l, device=dev).items()}
        t = lambda tag, shape, dtype="bf16": synth.tensor(w, (l,) + tag, shape, 1.0, 0, dev, dtype).double().cpu().numpy()
        H = t((1,), (nw, w.d))
        ls = {"K": t((2,), (w.n_pos, w.n_kv_heads, w.head_dim)), "V": t((3,), (w.n_pos, w.n_kv_heads, w.head_dim)),
              "P": t((4,), (w.n_clusters, w.n_heads, w.n_pos), "f32")}
        z, m, _ = O.spherical_kmeans(H, w.n_clusters, synth.kmeans_init(w, nw, l, 0), w.kmeans_iters)
        ls.update(Z=cfg.st(z), M=m)
        if w.resid != "raw":
            ls["codes"], ls["scales"] = O.residual_quantize(H, ls["Z"], m, w.resid)
        else:
            ls["H"] = H
        h_act = t((5,), (w.block, w.d))
        for _ in range(passes):
            t0 = time.perf_counter()
            cu = O.cluster_update(ls, cfg)
            dr = O.drift_layer(ls, W, cfg, blk, h_act, cu["h"], cu["patched"], True)
            rf = O.refresh_layer(W, cfg, h_act, cu["h"], dr["o"], dr["S"])
            t_total += time.perf_counter() - t0
            layers += 1
        del W
        if t_total >= budget_s:
            break
    per_step = t_total / layers * w.n_layers   # layers counts layer passes
    what = "window update, drift, sparse forward"
    if w.vocab:
        wlm = synth.weight(w, 0, "wlm", device=dev).double().cpu().numpy()
        t0 = time.perf_counter()
        rows = np.concatenate([rf["h_act_out"], rf["U"]], 0)
        c, _, _ = O.confidence(rows, wlm, w.vocab - 1, cfg.eps, cfg.st)
        O.commit_decide(np.zeros(w.block), c[: w.block], np.ones(w.block, bool), np.zeros((w.block, w.hist)),
                        np.zeros(w.block, np.int32), w.hist, w.alpha, w.tau_s)
        per_step += time.perf_counter() - t0
        what += "; the commit's LM head and decision once"
        del wlm
    return {"value": 1.0 / (per_step * w.batch), "unit": "refresh-steps/s", "cores": info["blas_threads"],
            "kind": "oracle", "cpu_model": info["cpu_model"], "host_cpus": info["host_cpus"],
            "sample": f"{layers // passes} of {w.n_layers} layers of one sequence's refresh step ({what}), "
                      f"{passes} passes each, {t_total:.1f} s of CPU time, scaled to {w.n_layers} layers x "
                      f"{w.batch} sequence(s)"}


def oracle_step_timing(names=("tiny_fp32_layer", "llada8b_layer"), reps: int = 3) -> dict:
    """Single-thread CPU oracle time of one refresh step of the single-layer workloads (window
    update, drift, sparse forward, and the next layer's K/V of the packet), median of reps."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import polestar_oracle as O
    out = {}
    with threadpool_limits(limits=1):
        for w in synth.WORKLOADS.values():
            if w.name not in names:
                continue
            cfg = O.Cfg.from_workload(w)
            blk = w.prompt
            nw = len(O.window_positions(blk, w.n_pos, w.block, w.win_prefix, w.win_suffix))
            W = {k: v.double().numpy() for k, v in synth.layer_weights(w, 0).items()}
            W1 = {k: v.double().numpy() for k, v in synth.layer_weights(w, 1).items()}
            t = lambda tag, shape, dt=w.dtype: synth.tensor(w, (0,) + tag, shape, 1.0, 0, "cpu", dt).double().numpy()
            H = t((1,), (nw, w.d))
            times = []
            for _ in range(reps):
                ls = {"K": t((2,), (w.n_pos, w.n_kv_heads, w.head_dim)),
                      "V": t((3,), (w.n_pos, w.n_kv_heads, w.head_dim)),
                      "P": t((4,), (w.n_clusters, w.n_heads, w.n_pos), "f32")}
                z, m, _ = O.spherical_kmeans(H, w.n_clusters, synth.kmeans_init(w, nw, 0, 0), w.kmeans_iters)
                ls.update(Z=cfg.st(z), M=m, H=H.copy())
                h_act = t((5,), (w.block, w.d))
                t0 = time.perf_counter()
                cu = O.cluster_update(ls, cfg)
                dr = O.drift_layer(ls, W, cfg, blk, h_act, cu["h"], cu["patched"], True)
                rf = O.refresh_layer(W, cfg, h_act, cu["h"], dr["o"], dr["S"])
                O.kv_rows(rf["U"], W1["wk"], W1["wv"], cfg)
                times.append(time.perf_counter() - t0)
            out[w.name] = {"seconds_per_step": float(np.median(times)), "reps": reps, "threads": 1,
                           "selected_rows": int(len(dr["S"]))}
    return {"oracle_single_thread": out, **host_info()}


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


WORKLOADS = {"llada8b_stack32": 3, "dream7b_gqa_stack28": 4, "llada8b_batch16_nvfp4_commit": 5}


def copy_bandwidth(torch, mib: int = 1024) -> float:
    """Measured device copy bandwidth: bytes read plus bytes written per second (GB/s) of a
    contiguous copy of `mib` MiB, the best of five."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(6):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        dst.copy_(src)
        ev1.record()
        torch.cuda.synchronize()
        best = min(best, ev0.elapsed_time(ev1))
    del src, dst
    return 2 * (mib << 20) / (best * 1e-3) / 1e9


def trajectory(w, bt, h_in, graph, graph_a, step, out):
    """The workload's own trajectory: its unmask schedule over its step count, each step a refresh
    or an active-only step as the update trigger decides (tau_upd), one event between steps."""
    import numpy as np
    import torch

    import synth
    from drift_driven_sparse_amd import binding as B
    sched = synth.unmask_schedule(w, steps=w.steps)
    tin = synth.tensor(w, (98,), (len(sched), bt, w.block, w.d), 1.0, 0, "cuda", "bf16")
    kinds, decoded = [], 0
    for _, offs in sched:
        decoded += len(offs)
        r = bool(B.polestar_should_refresh(decoded, w.tau_upd))
        decoded = 0 if r else decoded
        kinds.append(r)
    tev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sched) + 1)]
    torch.cuda.synchronize()
    tev[0].record()
    for t, r in enumerate(kinds):
        h_in.copy_(tin[t])
        if graph is not None:
            (graph if r else graph_a).replay()
        else:
            step(r)
        tev[t + 1].record()
    torch.cuda.synchronize()
    tper = np.array([tev[t].elapsed_time(tev[t + 1]) for t in range(len(kinds))])
    kr = np.array(kinds)
    out["trajectory"] = {
        "steps": len(kinds), "refresh_steps": int(kr.sum()), "active_only_steps": int((~kr).sum()),
        "tau_upd": w.tau_upd, "ms_total": round(float(tper.sum()), 3),
        "steps_per_s": round(1000.0 * len(kinds) / float(tper.sum()), 2),
        "refresh_ms_median": round(float(np.median(tper[kr])), 4) if kr.any() else None,
        "refresh_ms_mean": round(float(np.mean(tper[kr])), 4) if kr.any() else None,
        "active_only_ms_median": round(float(np.median(tper[~kr])), 4) if (~kr).any() else None,
        "active_only_ms_mean": round(float(np.mean(tper[~kr])), 4) if (~kr).any() else None}
    log(f"[bench] trajectory of {len(kinds)} steps ({int(kr.sum())} refresh): {tper.sum():.2f} ms")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llada8b_stack32", choices=list(WORKLOADS))
    ap.add_argument("--no-graph", action="store_true", help="launch every kernel from the host loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=None, help="(diagnostics) fewer layers than the workload")
    ap.add_argument("--entry", action="store_true",
                    help="time the block entry (polestar_entry, full and window kinds) instead of the step")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="also run one element-wise copy of MB MiB (reference for hardware byte counters)")
    ap.add_argument("--no-trajectory", action="store_true",
                    help="(diagnostics) skip the trajectory, so that a kernel trace holds refresh steps only")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="(CPU only) single-thread oracle time per refresh step of the single-layer workloads")
    args = ap.parse_args()
    if args.oracle_timing:
        print(json.dumps(oracle_step_timing()), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this refresh path runs on a single MI355X and uses no "
              "collectives; run it without --gpus or with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only (WORLD_SIZE > 1 refused).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from drift_driven_sparse_amd import binding as B
    from drift_driven_sparse_amd.stack import RefreshStack

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    w = synth.WORKLOADS[WORKLOADS[args.workload]]
    n_layers = args.layers or w.n_layers
    bt = w.batch
    commit = w.vocab > 0
    dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn, n_pos=w.n_pos,
                  batch=bt, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix,
                  n_clusters=w.n_clusters, top_k=w.top_k, vocab=w.vocab, dtype=B.BF16,
                  resid_fmt=B.RESID_BY_NAME[w.resid])
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist,
                      mask_id=max(w.vocab - 1, 0), kmeans_iters=w.kmeans_iters)
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
        rows = synth.tensor(w, (l, 12), (bt, nw, w.d), 1.0, 0, "cuda", "bf16")
        if "win_h" in L:
            L["win_h"].copy_(rows)
            rows = L["win_h"]
        entry_rows.append(rows)
        inits.append(torch.stack([torch.tensor(synth.kmeans_init(w, nw, l, 0, 0, b), dtype=torch.int32)
                                  for b in range(bt)]).cuda())
    if commit:
        st.set_lm_head(synth.weight(w, 0, "wlm", device="cuda"))
    torch.cuda.synchronize()
    log(f"[bench] {args.workload}: weights and state of {n_layers} layers, {bt} sequence(s), ready in "
        f"{time.time() - t0:.1f}s")
    if args.entry:
        # block entry of the whole stack from seeded layer-0 rows of every position
        h0 = torch.stack([synth.embeddings(w, 0, "cuda", b).to(torch.bfloat16) for b in range(bt)]).contiguous()
        res = entry_timing(st, w, blk, h0, inits, n_layers)
        st.close()
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle's block entry on a bounded sample")
            for name, full in (("full", True), ("window", False)):
                res[name]["cpu_baseline"] = entry_cpu_baseline(w, blk, full, budget_s=10.0)
        print(json.dumps({"metric": f"block entry ms ({w.name}), 1 GPU", "unit": "ms",
                          "higher_is_better": False, "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": f"{w.name}: {n_layers} layers, n {w.n_pos}, block start {blk}",
                                     "layers": n_layers, "batch": bt}, "block_entry": res}), flush=True)
        return
    # clustering of seeded window rows: the state a block entry leaves (the dense forward that
    # produces it is timed with --entry)
    st.block_entry(blk, entry_rows, inits)
    n_in = args.warmup + args.steps + 1
    inputs = synth.tensor(w, (99,), (n_in, bt, w.block, w.d), 1.0, 0, "cuda", "bf16")
    h_in = torch.zeros(bt, w.block, w.d, dtype=torch.bfloat16, device="cuda")

    def step(refresh=True):
        out = st.step(blk, h_in, refresh=refresh)
        if commit:
            st.commit(blk, out)

    # first refresh step establishes the drift references (proxy and active logits)
    h_in.copy_(inputs[0])
    step()
    torch.cuda.synchronize()

    graph = graph_a = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()          # eager run on the capture stream (lazy init)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph_a = torch.cuda.CUDAGraph()   # the active-only step (no refresh) of the trajectory
        with torch.cuda.graph(graph_a):
            step(False)
        torch.cuda.synchronize()
        log("[bench] refresh and active-only steps captured in HIP graphs")

    def run_step(i, eager=False):
        h_in.copy_(inputs[i])
        if graph is not None and not eager:
            graph.replay()
        else:
            step()

    for i in range(args.warmup):
        run_step(1 + i)
    torch.cuda.synchronize()
    if graph is None:
        B.polestar_profile(st.h, True)
    # timed region: K steps back to back, an event between consecutive steps (per-step times)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        run_step(1 + args.warmup + i, graph is None)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    ms_total = evs[0].elapsed_time(evs[-1])
    ms_step = ms_total / args.steps
    log(f"[bench] {args.steps} steps in {ms_total:.2f} ms ({ms_step:.3f} ms/step mean, median "
        f"{np.median(per):.3f}, graph={graph is not None})")
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
        spin_cycles = int(1_000_000 * 80.0 * max(1, bt // 4) / max(probe0.elapsed_time(probe1), 1e-3))
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

    # selected-row counts per layer and sequence (instrumented eager step, outside the timed region)
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
        counts.append(st.pk_cnt[l % 2].cpu().numpy().astype(np.float64))
        u_in, cur = sel, 1 - cur
    counts = np.stack(counts)                                   # [layers, batch]
    n_sel = float(counts.mean())
    step_bytes, step_flops = 0.0, 0.0
    for l in range(n_layers):
        lb = layer_bytes(w, float(counts[l].mean()), bt)
        step_bytes += sum(v for k, v in lb.items() if k != "gu_launch")
        n_patch = float(counts[l - 1].mean()) if l > 0 else 0.0
        step_flops += sum(layer_flops(w, float(counts[l].mean()), n_patch, bt).values())
    step_bytes += bt * 2 * 2 * 4 * w.block * w.n_heads * w.n_pos        # the last layer's active logits r/w
    suffix_sel = 0.0
    if commit:
        step_bytes += 2 * w.vocab * w.d
        suffix_sel = min(float(counts[-1].mean()), w.win_suffix)   # an upper bound: suffix rows of the last packet
        step_flops += bt * 2 * w.d * w.vocab * (w.block + suffix_sel)
    lb = layer_bytes(w, n_sel, bt)
    per_kind = {k: (v[0] / max(v[1], 1), v[1]) for k, v in prof.items() if v[1]}
    gu_ms, gu_n = per_kind.get("gu", (float("nan"), 0))
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    step_tfs = step_flops / (ms_step * 1e-3) / 1e12
    timing = ("HIP events around each launch of the kernel in an eager pass of the same step, queued behind a "
              "GPU spin so that the launches run back to back")
    if commit:
        gu_flops = 2 * w.d * 2 * w.ffn * (w.block + n_sel) * bt
        achieved = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "gate/up projection (bf16 GEMM with the SwiGLU product; split-K finish where split), all sequences",
                "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "flops_per_launch": gu_flops, "avg_launch_ms": round(gu_ms, 5), "launches": gu_n, "timing": timing}
    else:
        achieved = lb["gu_launch"] / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "gate/up projection (bf16 GEMM with the SwiGLU product; split-K finish where split)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic() if args.workload == "llada8b_stack32" else None,
                "bytes_per_launch": lb["gu_launch"], "avg_launch_ms": round(gu_ms, 5), "launches": gu_n,
                "timing": timing}
    kern = {k: {"avg_ms": round(v[0], 5), "launches": v[1]} for k, v in per_kind.items()}
    heads = f"{w.n_heads}x{w.head_dim} heads" if w.n_heads == w.n_kv_heads else \
        f"{w.n_heads}/{w.n_kv_heads} x{w.head_dim} GQA heads"
    out = {
        "metric": METRIC if args.workload == "llada8b_stack32" else
        f"drift-refresh steps/s ({w.name}) + % peak {'MFMA' if commit else 'HBM'}, 1 GPU",
        "value": round(1000.0 / ms_step, 3), "unit": "refresh-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "median_ms_per_step": round(float(np.median(per)), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {n_layers} layers, hidden {w.d}, {heads}, FFN {w.ffn}, "
                               f"prompt {w.prompt} + gen {w.gen}, B {w.block}, window {w.win_prefix}+{w.win_suffix}, "
                               f"K {w.n_clusters}, top-k {w.top_k}, batch {bt}, window storage {w.resid}"
                               + (f", commit over vocab {w.vocab}" if commit else ""),
                   "layers": n_layers, "n_pos": w.n_pos, "batch": bt, "graph": graph is not None,
                   "profiled_eager_ms_per_step": None if eager_ms_step is None else round(eager_ms_step, 4),
                   "mean_selected_rows": round(n_sel, 2)},
        "step_hbm": {"algorithmic_bytes": int(step_bytes), "achieved_GBs": round(step_gbs, 1),
                     "frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4)},
        "step_mfma": {"algorithmic_flops": int(step_flops), "achieved_TFLOPs": round(step_tfs, 2),
                      "frac_of_bf16_peak": round(step_tfs / MFMA_BF16_PEAK_TFLOPS, 4)},
        "roofline": roof,
        "kernels": kern,
        "copy_GBs": round(copy_bandwidth(torch), 1),
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
    if args.no_trajectory:
        out["trajectory"] = None
    else:
        trajectory(w, bt, h_in, graph, graph_a, step, out)
    st.close()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
