"""The layer stack in the launch configuration the benchmark times: one refresh
step of a LLaDA-8B-shaped stack (hidden 4096, 32 heads, FFN 12288, n 1024)
captured in a HIP graph.  Every replay must reproduce the eager step bit for
bit: the last layer's active rows, its drift outputs, every update packet and
all state the step leaves behind (K/V caches, window rows, centroids, proxy
and active logits).  The graph is replayed several times from the same saved
state, with eager work and synchronisations in between.  (Oracle parity of the
same kernels at these shapes is covered by the layer and trajectory tests.)
"""
from __future__ import annotations

import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from drift_driven_sparse_amd.stack import RefreshStack
from tests.harness import log

pytestmark = pytest.mark.gpu

STATE = ("k_cache", "v_cache", "win_h", "win_z", "win_m", "proxy_logits", "q_win", "q_ok")


def _snapshot(st: RefreshStack):
    snap = [{k: L[k].clone() for k in STATE} for L in st.layers]
    snap.append({"act_logits": st.act_logits.clone()})
    return snap


def _restore(st: RefreshStack, snap):
    for L, s in zip(st.layers, snap):
        for k in STATE:
            L[k].copy_(s[k])
    st.act_logits.copy_(snap[-1]["act_logits"])


def _outputs(st: RefreshStack, out_h: torch.Tensor):
    o = {"h_out": out_h.clone(), "D": st.D.clone(), "topk": st.topk.clone(), "delta": st.delta.clone()}
    for i in range(2):   # packet rows past the count are whatever an earlier step left there
        c = int(st.pk_cnt[i][0])
        o[f"pk_rows{i}"] = st.pk_rows[i][:, :c].clone()
        o[f"pk_idx{i}"] = st.pk_idx[i][:, :c].clone()
        o[f"pk_cnt{i}"] = st.pk_cnt[i].clone()
    for l, L in enumerate(st.layers):
        for k in STATE:
            o[f"{k}{l}"] = L[k].clone()
    o["act_logits"] = st.act_logits.clone()
    return o


def test_stack_graph_replay_matches_eager():
    w = synth.WORKLOADS[3]
    n_layers = 3
    dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn,
                  n_pos=w.n_pos, batch=1, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix,
                  n_clusters=w.n_clusters, top_k=w.top_k, vocab=0, dtype=B.BF16, resid_fmt=B.RESID_RAW)
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist, mask_id=0,
                      kmeans_iters=w.kmeans_iters)
    log(f"[stack] {n_layers} layers of {w.name}, n={w.n_pos}")
    st = RefreshStack(dims, params, n_layers)
    try:
        blk = w.prompt
        entry_rows, inits = [], []
        for l in range(n_layers):
            st.set_layer_weights(l, synth.layer_weights(w, l, device="cuda"))
            L = st.layers[l]
            L["k_cache"].copy_(synth.tensor(w, (l, 10), L["k_cache"].shape, 1.0, 0, "cuda", "bf16"))
            L["v_cache"].copy_(synth.tensor(w, (l, 11), L["v_cache"].shape, 1.0, 0, "cuda", "bf16"))
            L["win_h"].copy_(synth.tensor(w, (l, 12), L["win_h"].shape, 1.0, 0, "cuda", "bf16"))
            entry_rows.append(L["win_h"])
            inits.append(torch.tensor(synth.kmeans_init(w, st.win_max, l, 0), dtype=torch.int32, device="cuda")[None])
        st.block_entry(blk, entry_rows, inits)
        inputs = synth.tensor(w, (99,), (3, 1, w.block, w.d), 1.0, 0, "cuda", "bf16")
        h_in = torch.zeros(1, w.block, w.d, dtype=torch.bfloat16, device="cuda")
        h_in.copy_(inputs[0])
        st.step(blk, h_in)                      # first step: drift references
        torch.cuda.synchronize()
        snap = _snapshot(st)
        h_in.copy_(inputs[1])
        out = st.step(blk, h_in)
        torch.cuda.synchronize()
        want = _outputs(st, out)
        log(f"[stack] eager step: selected rows per packet {[int(want[f'pk_cnt{i}'][0]) for i in range(2)]}, "
            f"topk {want['topk'].tolist()}")
        # capture on a side stream after a warm eager run there
        _restore(st, snap)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            st.step(blk, h_in)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gout = st.step(blk, h_in)
        torch.cuda.synchronize()
        for rep in range(3):
            _restore(st, snap)
            h_in.copy_(inputs[1])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = _outputs(st, gout)
            bad = [k for k in want if not torch.equal(got[k], want[k])]
            log(f"[stack] replay {rep}: {len(want) - len(bad)}/{len(want)} tensors bit-identical")
            assert not bad, f"replay {rep} differs from the eager step in {bad}"
            # eager work between replays
            h_in.copy_(inputs[2])
            st.step(blk, h_in)
            torch.cuda.synchronize()
    finally:
        st.close()
    log("[stack] graph replays match the eager step")


@pytest.mark.parametrize("refresh", [True, False])
def test_step_call_matches_layer_calls(refresh):
    """polestar_step (one call for the whole stack) against the stack's per-layer calls from the
    same saved state: every output and all state left behind bit for bit."""
    w = synth.shrink(synth.WORKLOADS[1], dtype="bf16")
    n_layers = 3
    dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn,
                  n_pos=w.n_pos, batch=2, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix,
                  n_clusters=w.n_clusters, top_k=w.top_k, vocab=0, dtype=B.BF16, resid_fmt=B.RESID_RAW)
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist, mask_id=0,
                      kmeans_iters=w.kmeans_iters)
    log(f"[step-call] {n_layers} layers of {w.name} (bf16, batch 2), refresh={refresh}")
    st = RefreshStack(dims, params, n_layers)
    try:
        blk = w.prompt
        entry_rows, inits = [], []
        for l in range(n_layers):
            st.set_layer_weights(l, synth.layer_weights(w, l, device="cuda"))
            L = st.layers[l]
            L["k_cache"].copy_(synth.tensor(w, (l, 10), L["k_cache"].shape, 1.0, 0, "cuda", "bf16"))
            L["v_cache"].copy_(synth.tensor(w, (l, 11), L["v_cache"].shape, 1.0, 0, "cuda", "bf16"))
            L["win_h"].copy_(synth.tensor(w, (l, 12), L["win_h"].shape, 1.0, 0, "cuda", "bf16"))
            entry_rows.append(L["win_h"])
            inits.append(torch.stack([torch.tensor(synth.kmeans_init(w, st.win_max, l, 0, 0, b), dtype=torch.int32)
                                      for b in range(2)]).cuda())
        st.block_entry(blk, entry_rows, inits)
        inputs = synth.tensor(w, (99,), (2, 2, w.block, w.d), 1.0, 0, "cuda", "bf16")
        st.step(blk, inputs[0])                 # drift references
        torch.cuda.synchronize()
        snap = _snapshot(st)
        out = st.step(blk, inputs[1], refresh=refresh, per_layer=True)
        torch.cuda.synchronize()
        want = _outputs(st, out)
        _restore(st, snap)
        st.h_act[0].copy_(inputs[1])
        mode = B.DRIFT_REFRESH if refresh else B.DRIFT_ACTIVE_ONLY
        B.polestar_step(st.h, mode, [st.struct(l) for l in range(n_layers)], blk, st.h_act[0], st.h_act[1],
                        st.packets[0], st.packets[1], st.D, st.topk, st.act_logits, st.delta, st.ws, st.ws_bytes)
        torch.cuda.synchronize()
        got = _outputs(st, st.h_act[n_layers % 2])
        bad = [k for k in want if not torch.equal(got[k], want[k])]
        log(f"[step-call] {len(want) - len(bad)}/{len(want)} tensors bit-identical")
        assert not bad, f"polestar_step differs from the per-layer calls in {bad}"
    finally:
        st.close()


def test_query_cache_matches_full_projection():
    """The window-row query cache (raw window rows: only patched rows projected after the first
    refresh of a block) against a stack that projects every window row: bit-identical outputs and
    state over a block entry and five steps, then a full and a window entry of the next block with
    steps after each (the entry clears the cache: q_ok 0 after it, blk_start + 1 after the first
    refresh), and a refresh at a later block position with no entry (a stale tag: every window row
    is projected again)."""
    w = synth.shrink(synth.WORKLOADS[1], dtype="bf16")
    n_layers = 3
    dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn,
                  n_pos=w.n_pos, batch=2, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix,
                  n_clusters=w.n_clusters, top_k=w.top_k, vocab=0, dtype=B.BF16, resid_fmt=B.RESID_RAW)
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist, mask_id=0,
                      kmeans_iters=w.kmeans_iters)
    blk0 = w.prompt
    nw = w.win_prefix + w.win_suffix
    stacks = [RefreshStack(dims, params, n_layers, q_cache=qc) for qc in (True, False)]
    # (kind, block start, refresh): "e" full entry, "w" window entry, "s" step
    plan = [("e", blk0, None)] + [("s", blk0, r) for r in (True, True, False, True, True)]
    blk1, blk2 = blk0 + w.block, blk0 + 2 * w.block
    plan += [("e", blk1, None), ("s", blk1, True), ("s", blk1, False), ("s", blk1, True)]
    plan += [("w", blk1, None), ("s", blk1, True), ("s", blk1, True)]
    plan += [("s", blk2, True), ("s", blk2, True)]
    try:
        h0 = torch.stack([synth.embeddings(w, 0, "cuda", b).to(torch.bfloat16) for b in range(2)]).contiguous()
        inits = [torch.stack([torch.tensor(synth.kmeans_init(w, nw, l, 0, 0, b), dtype=torch.int32)
                              for b in range(2)]).cuda() for l in range(n_layers)]
        inputs = synth.tensor(w, (98,), (len(plan), 2, w.block, w.d), 1.0, 0, "cuda", "bf16")
        outs, tags = [], []
        for si, st in enumerate(stacks):
            for l in range(n_layers):
                st.set_layer_weights(l, synth.layer_weights(w, l, device="cuda"))
            seq, tg = [], []
            h_seq = h0
            for i, (kind, blk, refresh) in enumerate(plan):
                if kind in ("e", "w"):
                    out = st.entry_forward(blk, h_seq, inits, full=kind == "e").clone()
                    torch.cuda.synchronize()
                    seq.append([out] + [L[k].clone() for L in st.layers for k in ("k_cache", "v_cache", "win_h",
                                                                                     "win_z", "proxy_logits")])
                else:
                    out = st.step(blk, inputs[i], refresh=refresh)
                    torch.cuda.synchronize()
                    seq.append([out.clone(), st.D.clone(), st.topk.clone(), st.delta.clone()] +
                               [L[k].clone() for L in st.layers for k in ("k_cache", "v_cache", "win_h", "win_z",
                                                                             "proxy_logits")])
                if si == 0:
                    tg.append([int(L["q_ok"][b]) for L in st.layers for b in range(2)])
            outs.append(seq)
            tags = tags or tg
        # the tag each layer's cache should carry after every item of the plan
        cur = 0
        for i, (kind, blk, refresh) in enumerate(plan):
            if kind in ("e", "w"):
                cur = 0
            elif refresh:
                cur = blk + 1
            assert tags[i] == [cur] * (2 * n_layers), f"item {i} {plan[i]}: q_ok {tags[i]}, want {cur}"
        for i, (a, b_) in enumerate(zip(*outs)):
            bad = [j for j, (x, y) in enumerate(zip(a, b_)) if not torch.equal(x, y)]
            log(f"[q-cache] {plan[i]}: {len(a) - len(bad)}/{len(a)} tensors bit-identical")
            assert not bad, f"item {i} {plan[i]}: the query cache changes tensors {bad}"
    finally:
        for st in stacks:
            st.close()
