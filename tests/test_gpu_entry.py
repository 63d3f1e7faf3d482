"""Parity of the block-entry call (polestar_entry) with the CPU oracle.

For each case the GPU runs polestar_entry on one or two layers from seeded
hidden rows and a seeded stale cache; the oracle runs the same rows through
layer_forward_rows on the same stale cache, then block_entry_layer_state
(spherical k-means of the window rows of the layer input, residual codes,
proxy logits of the centroids over the fresh cache).  Compared:
  * the recomputed rows of h_out and of the K/V caches (stored values within
    the storage-dtype bounds), every other row bit-identical to what it held;
  * k-means labels and residual codes bit-exact, centroids within the bounds;
  * the proxy logits and (last layer) the active block's attention logits
    within 2e-3 (each side from its own stored cache and centroids).
A second layer takes each side's own first-layer output, so its values are
compared as free-running values.
"""
import numpy as np
import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O
from tests import flips as FL
from tests.harness import (LOGIT_FLOOR, Dev, assert_close, assert_derived, assert_stored, assert_traj, layer_struct, log, np64, oracle_weights,
                           packed_layer, weights)

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS[1]
CASES = {
    # name: (workload, batch, layers, full, blk_start)
    "tiny_fp32_full_2layers": (TINY, 1, 2, True, 64),
    "tiny_fp32_window": (TINY, 1, 1, False, 160),
    "tiny_bf16_full_2layers_batch2": (synth.shrink(TINY, dtype="bf16"), 2, 2, True, 96),
    "tiny_bf16_full_2layers_proxy_active": (synth.shrink(TINY, dtype="bf16", proxy_support="active"), 1, 2, True, 96),
    "tiny_fp32_window_proxy_active": (synth.shrink(TINY, proxy_support="active"), 1, 1, False, 160),
    "tiny_bf16_window_at_start": (synth.shrink(TINY, dtype="bf16"), 1, 1, False, 0),
    "tiny_bf16_window_at_end": (synth.shrink(TINY, dtype="bf16"), 1, 1, False, 288),
    "tiny_bf16_nvfp4_full": (synth.shrink(TINY, dtype="bf16", resid="nvfp4"), 1, 1, True, 128),
    "tiny_bf16_mxfp4_window_batch2": (synth.shrink(TINY, dtype="bf16", resid="mxfp4"), 2, 1, False, 128),
    "small_window_B8": (synth.shrink(TINY, dtype="bf16", prompt=32, gen=96, n_clusters=4, top_k=2, block=8,
                                     win_prefix=8, win_suffix=0), 1, 1, False, 48),
    "llada_layer_full": (synth.WORKLOADS[2], 1, 1, True, 512),
    "llada_n1024_full": (synth.shrink(synth.WORKLOADS[3], n_layers=1), 1, 1, True, 512),
    "dream_gqa_window": (synth.shrink(synth.WORKLOADS[4], n_layers=1), 1, 1, False, 384),
    # the batched NVFP4 workload at its full size: every sequence runs, the first and last are checked
    "llada_nvfp4_batch16_full_sampled": (synth.shrink(synth.WORKLOADS[5], n_layers=1, vocab=0), 16, 1, True, 512),
}
SAMPLED = {"llada_nvfp4_batch16_full_sampled": (0, 15)}


def _cache_pair(w, batch, run, seqs):
    """Seeded stale K/V caches (device layouts) and the oracle copies [n, Hkv, dh] of sequences seqs."""
    n, hkv, dh = w.n_pos, w.n_kv_heads, w.head_dim
    ks = [synth.tensor(w, (b, 30), (n, hkv, dh), 1.0, run, "cuda", w.dtype) for b in range(batch)]
    vs = [synth.tensor(w, (b, 31), (n, hkv, dh), 1.0, run, "cuda", w.dtype) for b in range(batch)]
    kc = torch.stack(ks).contiguous()
    vc = torch.stack([v.permute(1, 2, 0) for v in vs]).contiguous()
    return kc, vc, {b: np64(ks[b]) for b in seqs}, {b: np64(vs[b]) for b in seqs}


@pytest.mark.parametrize("case", list(CASES))
def test_block_entry_parity(case):
    w, batch, n_layers, full, blk_start = CASES[case]
    log(f"[entry] case={case} d={w.d} n={w.n_pos} heads={w.n_heads}/{w.n_kv_heads} batch={batch} dtype={w.dtype} "
        f"resid={w.resid} layers={n_layers} mode={'full' if full else 'window'} blk_start={blk_start}")
    dev = Dev(w, batch=batch, vocab=0)
    cfg = O.Cfg.from_workload(w)
    st = cfg.st
    n, d, hq, hkv, dh, K, WM = w.n_pos, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.n_clusters, dev.win_max
    nv = w.resid != "raw"
    wpos = O.window_positions(blk_start, n, w.block, w.win_prefix, w.win_suffix)
    nw = len(wpos)
    keff = min(K, nw)
    rows = O.entry_positions(blk_start, n, w.block, w.win_prefix, w.win_suffix, full)
    others = np.setdiff1d(np.arange(n), rows)
    cb, sb = B.polestar_resid_bytes(B.RESID_BY_NAME[w.resid], d) if nv else (0, 0)
    mode = B.ENTRY_FULL if full else B.ENTRY_WINDOW

    # layer inputs: seeded rows for every position, rounded to the storage dtype
    h_in = torch.stack([synth.embeddings(w, 0, "cuda", b).to(dev.tdt) for b in range(batch)]).contiguous()
    h_or = {b: np64(h_in[b]) for b in SAMPLED.get(case, range(batch))}
    for l in range(n_layers):
        W = weights(w, l)
        P = packed_layer(dev, W)
        Wo = oracle_weights(W)
        del W
        kc, vc, k_or, v_or = _cache_pair(w, batch, l, SAMPLED.get(case, range(batch)))
        kc0, vc0 = kc.clone(), vc.clone()
        z = dev.zeros(batch, K, d)
        m = torch.zeros(batch, WM, dtype=torch.int32, device="cuda")
        plog = torch.full((batch, K, hq, n), 7.0, dtype=torch.float32, device="cuda")
        init = torch.zeros(batch, K, dtype=torch.int32, device="cuda")
        inits = [synth.kmeans_init(w, nw, l, 0, 0, b) for b in range(batch)]
        for b in range(batch):
            init[b, :keff] = torch.tensor(inits[b])
        Ld = dict(P, k_cache=kc, v_cache=vc, win_z=z, win_m=m, proxy_logits=plog)
        if nv:
            codes = torch.zeros(batch, WM, cb, dtype=torch.uint8, device="cuda")
            scales = torch.zeros(batch, WM, max(sb, 1), dtype=torch.uint8, device="cuda")
            Ld.update(win_codes=codes, win_scales=scales)
        else:
            win = dev.zeros(batch, WM, d)
            Ld.update(win_h=win)
        h_out = torch.full_like(h_in, 3.0)
        obj = torch.zeros(batch, 2 * w.kmeans_iters, dtype=torch.float64, device="cuda")
        last = l == n_layers - 1
        act = torch.full((batch, w.block, hq, n), 5.0, dtype=torch.float32, device="cuda") if last else None
        B.polestar_entry(dev.h, mode, layer_struct(Ld), blk_start, h_in, init, h_out, obj, act, dev.ws,
                         dev.ws_bytes)
        torch.cuda.synchronize()
        log(f"[entry] layer {l}: GPU done")
        cmp_rows = assert_stored if l == 0 else (lambda a, b_, dt, name: assert_traj(a, b_, dt, name))
        nxt = {}
        for b in SAMPLED.get(case, range(batch)):
            Kb, Vb = k_or[b].copy(), v_or[b].copy()
            out_or = O.layer_forward_rows(h_or[b][rows], rows, Wo, cfg, Kb, Vb)
            ls = O.block_entry_layer_state(h_or[b], Kb, Vb, Wo["wq"], cfg, blk_start, inits[b])
            # recomputed rows and cache rows; the rest untouched
            cmp_rows(np64(h_out[b, rows]), out_or, w.dtype, f"layer {l} seq {b} outputs")
            assert torch.all(h_out[b, others] == 3.0), "rows outside the entry set were written"
            kg = np64(kc[b]).reshape(n, -1)
            vg = np64(vc[b].permute(2, 0, 1)).reshape(n, -1)
            cmp_rows(kg[rows], Kb.reshape(n, -1)[rows], w.dtype, f"layer {l} seq {b} K rows")
            cmp_rows(vg[rows], Vb.reshape(n, -1)[rows], w.dtype, f"layer {l} seq {b} V rows")
            assert torch.equal(kc[b, others], kc0[b, others]), "K rows outside the entry set changed"
            assert torch.equal(vc[b][..., others], vc0[b][..., others]), "V rows outside the entry set changed"
            # clustering of the window rows of this layer's input (each side's own input rows)
            if l == 0:
                assert np.array_equal(m[b, :nw].cpu().numpy(), ls["M"]), "k-means labels differ"
                assert np.allclose(obj[b].cpu().numpy(), ls["trace"], rtol=1e-12, atol=0), "k-means objective"
                assert_stored(np64(z[b]), ls["Z"], w.dtype, "entry centroids")
                if nv:
                    assert np.array_equal(codes[b, :nw].cpu().numpy(), ls["codes"]), f"entry {w.resid} codes differ"
                    assert np.array_equal(scales[b, :nw, :sb].cpu().numpy(), ls["scales"])
                else:
                    assert torch.equal(win[b, :nw], h_in[b, wpos]), "window rows not stored as they are"
            else:
                # each side clusters its own input rows, which differ where a storage rounding went
                # the other way: labels must agree except at rows whose oracle cosine margin (best
                # against second-best centroid) is below 1e-3, reported
                xh = O.unit_rows(h_or[b][wpos])
                cos = np.sort(xh @ O.unit_rows(ls["Z"][:min(K, nw)]).T, axis=1)
                margin = cos[:, -1] - cos[:, -2] if cos.shape[1] > 1 else np.full(nw, np.inf)
                diff = np.nonzero(m[b, :nw].cpu().numpy() != ls["M"])[0]
                if len(diff):
                    log(f"    layer {l} seq {b}: {len(diff)} labels differ at oracle margins {margin[diff]}")
                assert np.all(margin[diff] < 1e-3), "k-means labels differ away from a near-tie"
                if not len(diff):
                    assert_derived(np64(z[b]), ls["Z"], w.dtype, f"layer {l} seq {b} entry centroids")
            # proxy logits (over the proxy keys) and, last layer, the active block's logits over the
            # fresh cache, against the oracle's own state: per-call rule on the first layer, whose
            # inputs both sides share; later layers start from each side's own stored rows
            pk = O.proxy_keys(cfg, blk_start)
            jpos = O.active_positions(blk_start, w.block)
            if l == 0:
                # admissible deviations from the oracle alone: the K/V rows and centroids this call
                # stores, and the rounded projection inputs
                hr = h_or[b][rows]
                dK, dV = np.zeros((n, hkv, dh)), np.zeros((n, hkv, dh))
                dnr = FL.norm_in_dev(hr, cfg.eps, w.dtype)
                for arr, wm in ((dK, Wo["wk"]), (dV, Wo["wv"])):
                    arr[rows] = FL.stored_dev(O.project(hr, wm, cfg.eps, st), w.dtype,
                                              FL.proj_dev(dnr, wm)).reshape(-1, hkv, dh)
                z_pre, _, _ = O.spherical_kmeans(h_or[b][wpos], K, inits[b], w.kmeans_iters)
                dz = FL.norm_in_dev(ls["Z"], cfg.eps, w.dtype, FL.stored_dev(z_pre, w.dtype))
                q_px = O.project(ls["Z"], Wo["wq"], cfg.eps, st).reshape(K, hq, dh)
                dlp = FL.attn_dev(q_px, Kb, Vb, FL.proj_dev(dz, Wo["wq"]).reshape(K, hq, dh), dK, dV, hq, hkv,
                                  keys=pk)[0]
                assert_close(plog[b].cpu().numpy()[..., pk], ls["P"][..., pk], f"layer {l} seq {b} proxy logits",
                             dtype=w.dtype, allow=dlp, floor=LOGIT_FLOOR)
            else:
                assert_derived(plog[b].cpu().numpy()[..., pk], ls["P"][..., pk], w.dtype,
                               f"layer {l} seq {b} proxy logits")
            if last:
                qa = O.project(h_or[b][jpos], Wo["wq"], cfg.eps, st).reshape(-1, hq, dh)
                _, lo = O.attention(qa, Kb, Vb, hq, hkv)
                if l == 0:
                    dqa = FL.proj_dev(FL.norm_in_dev(h_or[b][jpos], cfg.eps, w.dtype), Wo["wq"]).reshape(-1, hq, dh)
                    dla = FL.attn_dev(qa, Kb, Vb, dqa, dK, dV, hq, hkv)[0]
                    assert_close(act[b].cpu().numpy(), lo, f"seq {b} active logits", dtype=w.dtype, allow=dla,
                                 floor=LOGIT_FLOOR)
                else:
                    assert_derived(act[b].cpu().numpy(), lo, w.dtype, f"seq {b} active logits")
            hn = h_or[b].copy()
            hn[rows] = out_or
            nxt[b] = hn
        # every sequence (sampled or not): finite recomputed rows, labels inside [0, K)
        assert torch.isfinite(h_out[:, rows].float()).all(), "non-finite entry outputs"
        assert int(m[:, :nw].min()) >= 0 and int(m[:, :nw].max()) < K
        log(f"[entry] layer {l} ok")
        # the next layer continues from each side's own outputs
        h_in = h_out.clone()
        h_or = nxt
        del P, Ld
    dev.close()
    log(f"[entry] case={case} passed")


def test_entry_graph_replay_matches_eager():
    """The block entry of a 2-layer stack captured in a HIP graph: every replay (with eager work
    between replays) gives the eager entry's state bit for bit."""
    from drift_driven_sparse_amd.stack import RefreshStack
    w = synth.shrink(TINY, dtype="bf16", resid="nvfp4")
    dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn, n_pos=w.n_pos,
                  batch=2, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix, n_clusters=w.n_clusters,
                  top_k=w.top_k, vocab=0, dtype=B.BF16, resid_fmt=B.RESID_NVFP4)
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist, mask_id=0,
                      kmeans_iters=w.kmeans_iters)
    st = RefreshStack(dims, params, 2)
    try:
        blk = 96
        nw = len(O.window_positions(blk, w.n_pos, w.block, w.win_prefix, w.win_suffix))
        inits = []
        for l in range(2):
            st.set_layer_weights(l, synth.layer_weights(w, l, device="cuda"))
            inits.append(torch.stack([torch.tensor(synth.kmeans_init(w, nw, l, 0, 0, b), dtype=torch.int32)
                                      for b in range(2)]).cuda())
        h0 = torch.stack([synth.embeddings(w, 0, "cuda", b).to(torch.bfloat16) for b in range(2)]).contiguous()
        names = ("k_cache", "v_cache", "win_codes", "win_scales", "win_z", "win_m", "proxy_logits")

        def state(out):
            return [out.clone(), st.act_logits.clone()] + [L[k].clone() for L in st.layers for k in names]

        want = state(st.entry_forward(blk, h0, inits, full=True))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            st.entry_forward(blk, h0, inits, full=True)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gout = st.entry_forward(blk, h0, inits, full=True)
        for rep in range(3):
            st.act_logits.zero_()
            for L in st.layers:
                for k in names:
                    L[k].zero_()
            g.replay()
            torch.cuda.synchronize()
            got = state(gout)
            bad = [i for i, (a, b_) in enumerate(zip(got, want)) if not torch.equal(a, b_)]
            log(f"[entry-graph] replay {rep}: {len(want) - len(bad)}/{len(want)} tensors bit-identical")
            assert not bad, f"replay {rep} differs from the eager entry in tensors {bad}"
            st.entry_forward(blk, h0, inits, full=False)   # eager work between replays
            torch.cuda.synchronize()
    finally:
        st.close()
