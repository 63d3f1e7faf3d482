"""Per-call parity of one layer's refresh step: HIP path vs the CPU oracle on the
same seeded inputs.

Each case builds synthetic layer state (KV caches, window rows, an update
packet, the previous logits), runs on the GPU
  cluster(ENTRY) -> cluster(UPDATE, packet) -> drift(REFRESH) -> refresh(+ next-layer K/V)
  -> cluster(UPDATE) of layer l+1 with the new packet,
and after every call compares against the oracle run on the identical inputs.
Discrete outputs (labels, top-k, S, residual codes) must match exactly; floating
point values before their storage rounding must match within 2e-3 relative.
Where the GPU's pre-rounding value is available (check copies), its stored
value must be exactly that value rounded once; stored values whose inputs are
identical on both sides must also stay within the bounds of the oracle's stored
values.  The next layer's K/V rows are projections of each side's own stored
update packet, so there only the pre-rounding values are compared with the
oracle.
"""
import math

import numpy as np
import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O
from tests import flips as FL
from tests.harness import (LOGIT_FLOOR, row_err, check_topk, Dev, assert_close, assert_derived, assert_rounded,
                           assert_stored, layer_struct, log, np64, oracle_weights, packed_layer, packet, to_dev, topk_margin, weights)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, batch, overrides)
    "tiny_fp32": (synth.WORKLOADS[1], 1, {}),
    "tiny_fp32_k8": (synth.WORKLOADS[1], 1, {"top_k": 8}),
    "llada_layer_bf16": (synth.WORKLOADS[2], 1, {}),
    "llada_layer_n1024": (synth.WORKLOADS[3], 1, {}),
    "dream_gqa_layer": (synth.WORKLOADS[4], 1, {}),
    "llada_nvfp4_batch2": (synth.WORKLOADS[5], 2, {}),
    "tiny_bf16_window_tail": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=64, gen=64), 1,
                              {"blk_start": 96}),
    "tiny_bf16_small_window": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=4, gen=64), 1,
                               {"blk_start": 4}),
    # sweep ranges of the page's ablations: clusters K, selected clusters k, block B, window (p, s)*B
    "sweep_K4_k2_B8_w10": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=128, n_clusters=4,
                                        top_k=2, block=8, win_prefix=8, win_suffix=0), 1, {}),
    "sweep_K16_k6_B16_w21": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=128, n_clusters=16,
                                          top_k=6, block=16, win_prefix=32, win_suffix=16), 1, {}),
    "sweep_K16_k8_B64_w10": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=128, n_clusters=16,
                                          top_k=8, block=64, win_prefix=64, win_suffix=0), 1, {}),
    "sweep_K8_k4_B16_w31": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=128, block=16,
                                         win_prefix=48, win_suffix=16), 1, {}),
    "sweep_K8_k4_B32_w31": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=256,
                                         win_prefix=96, win_suffix=32), 1, {}),
    # 188 rows per sequence: the widest row tiling of every kernel
    "rows188_K4_k2_B64": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=256, n_clusters=4,
                                       top_k=2, block=64, win_prefix=96, win_suffix=24), 1, {}),
    # fewer window rows than clusters (n_Omega = 4 < K = 8): block entry and top-k over 4 clusters
    "tiny_bf16_nwin4_K8": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=4, gen=32), 1, {"blk_start": 4}),
    # windows (1,1)B and (2,2)B of the window ablation
    "sweep_B32_w11": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=256, win_prefix=32,
                                   win_suffix=32), 1, {}),
    "sweep_B32_w22": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=256, win_prefix=64,
                                   win_suffix=64), 1, {}),
    # more rows per sequence than one 192-row projection slab: B = 64 at the default (2,1)B window
    # (264 rows), and 336 rows with K = 16 at (3,1)B
    "rows264_B64_w21": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=256, gen=256, block=64,
                                     win_prefix=128, win_suffix=64), 1, {}),
    "rows336_K16_k8_B64_w31": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=256, gen=256, block=64,
                                            n_clusters=16, top_k=8, win_prefix=192, win_suffix=64), 1, {}),
    "llada_layer_B64_w21": (synth.shrink(synth.WORKLOADS[2], block=64, win_prefix=128, win_suffix=64), 1, {}),
    # more than 1024 positions (KL rows of 2048 and 4096 logits)
    "npos2048_bf16": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=1024, gen=1024), 1, {}),
    "npos4096_bf16": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=2048, gen=2048), 1, {}),
    # residual formats of the quantisation ablation
    "resid_fp8": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=128, resid="fp8"), 1, {}),
    "resid_mxint8": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=128, resid="mxint8"), 1, {}),
    "resid_mxfp4_batch2": (synth.shrink(synth.WORKLOADS[2], d=512, n_heads=4, n_kv_heads=4, ffn=1536, prompt=128,
                                        gen=128, resid="mxfp4"), 2, {}),
    # proxy attention over the active block's keys only (the other reading of the key support)
    "tiny_fp32_proxy_active": (synth.shrink(synth.WORKLOADS[1], proxy_support="active"), 1, {}),
    "llada_layer_proxy_active": (synth.shrink(synth.WORKLOADS[2], proxy_support="active"), 1, {}),
    "tiny_bf16_proxy_active_unaligned": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=100, gen=96,
                                                      proxy_support="active"), 1, {"blk_start": 132}),
}


def _state(w, dev, seq, nw, run=0):
    d, n, hkv, dh, hq = w.d, w.n_pos, w.n_kv_heads, w.head_dim, w.n_heads
    t = lambda tag, shape, std=1.0, dtype=w.dtype: synth.tensor(w, (seq,) + tag, shape, std, run, "cuda", dtype)
    s = {
        "K": t((10,), (n, hkv, dh)), "V": t((11,), (n, hkv, dh)),
        "K1": t((12,), (n, hkv, dh)), "V1": t((13,), (n, hkv, dh)),
        "H": t((14,), (nw, d)), "H1": t((15,), (nw, d)),
        "h_act": t((16,), (w.block, d)),
        "act_prev": t((17,), (w.block, hq, n), 1.0, "f32"),
    }
    rng = np.random.default_rng([w.seed(run), 99, seq])
    n_patch = min(nw, max(1, nw // 4))
    s["u_idx"] = np.sort(rng.choice(nw, size=n_patch, replace=False)).astype(np.int32)
    s["u_rows"] = t((18,), (n_patch, d))
    s["init"] = synth.kmeans_init(w, nw, 0, 0, run, seq)
    s["init1"] = synth.kmeans_init(w, nw, 1, 0, run, seq)
    return s


@pytest.mark.parametrize("case", list(CASES))
def test_layer_step_parity(case):
    w, batch, over = CASES[case]
    top_k = over.get("top_k")
    if top_k:
        w = synth.shrink(w, top_k=top_k)
    log(f"[layer-parity] case={case} d={w.d} n={w.n_pos} heads={w.n_heads}/{w.n_kv_heads} batch={batch} "
        f"dtype={w.dtype} resid={w.resid}")
    torch.manual_seed(0)
    dev = Dev(w, batch=batch, vocab=0)
    cfg = O.Cfg.from_workload(w, top_k=w.top_k)
    st = cfg.st
    n, d, hq, hkv, dh, Bk = w.n_pos, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.block
    blk_start = over.get("blk_start", w.prompt)
    wpos = O.window_positions(blk_start, n, Bk, w.win_prefix, w.win_suffix)
    nw, WM, K = len(wpos), dev.win_max, w.n_clusters
    keff = min(K, nw)
    nv = w.resid != "raw"   # window rows stored as residual codes
    W0, W1 = weights(w, 0), weights(w, 1)
    P0 = packed_layer(dev, W0)
    wkv1 = dev.pack(B.W_KV, torch.cat([W1["wk"], W1["wv"]], 0))
    Wo = oracle_weights(W0)
    wk1, wv1 = np64(W1["wk"]), np64(W1["wv"])
    del W1

    S = [_state(w, dev, b, nw) for b in range(batch)]
    # ---- device buffers
    kc = torch.stack([s["K"] for s in S]).contiguous()
    vc = torch.stack([s["V"].permute(1, 2, 0) for s in S]).contiguous()      # V cache: [Hkv, dh, n]
    kc1 = torch.stack([s["K1"] for s in S]).contiguous()
    vc1 = torch.stack([s["V1"].permute(1, 2, 0) for s in S]).contiguous()
    win = dev.zeros(batch, WM, d)
    win1 = dev.zeros(batch, WM, d)
    for b, s in enumerate(S):
        win[b, :nw] = s["H"]
        win1[b, :nw] = s["H1"]
    cb, sb = B.polestar_resid_bytes(B.RESID_BY_NAME[w.resid], d) if nv else (d // 2, d // 16)
    codes = torch.zeros(batch, WM, cb, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(batch, WM, max(sb, 1), dtype=torch.uint8, device="cuda")
    codes1, scales1 = codes.clone(), scales.clone()
    z = dev.zeros(batch, K, d)
    z1 = dev.zeros(batch, K, d)
    m = torch.zeros(batch, WM, dtype=torch.int32, device="cuda")
    m1 = m.clone()
    plog = torch.zeros(batch, K, hq, n, dtype=torch.float32, device="cuda")
    init = torch.zeros(batch, K, dtype=torch.int32, device="cuda")
    init1 = init.clone()
    for b, s in enumerate(S):
        init[b, :keff] = torch.tensor(s["init"])
        init1[b, :keff] = torch.tensor(s["init1"])
    obj = torch.zeros(batch, 2 * w.kmeans_iters, dtype=torch.float64, device="cuda")
    L0 = dict(P0, k_cache=kc, v_cache=vc, win_z=z, win_m=m, proxy_logits=plog)
    L1 = dict(k_cache=kc1, v_cache=vc1, win_z=z1, win_m=m1)
    if nv:
        L0.update(win_codes=codes, win_scales=scales)
        L1.update(win_codes=codes1, win_scales=scales1)
    else:
        L0.update(win_h=win)
        L1.update(win_h=win1)
    Ls0, Ls1 = layer_struct(L0), layer_struct(L1)

    # ---- 1. block-entry clustering of layers l and l+1
    B.polestar_cluster(dev.h, B.CLUSTER_ENTRY, Ls0, blk_start, None, init, win, obj, dev.ws, dev.ws_bytes)
    B.polestar_cluster(dev.h, B.CLUSTER_ENTRY, Ls1, blk_start, None, init1, win1, None, dev.ws, dev.ws_bytes)
    torch.cuda.synchronize()
    OL, OL1 = [], []
    for b, s in enumerate(S):
        Hb = np64(s["H"])
        zo, mo, tr = O.spherical_kmeans(Hb, K, s["init"], w.kmeans_iters)
        assert np.array_equal(m[b, :nw].cpu().numpy(), mo), "k-means labels differ"
        assert_stored(np64(z[b]), st(zo), w.dtype, "entry centroids")
        assert np.allclose(obj[b].cpu().numpy(), tr, rtol=1e-12, atol=0), "k-means objective trace"
        zo1, mo1, _ = O.spherical_kmeans(np64(s["H1"]), K, s["init1"], w.kmeans_iters)
        assert np.array_equal(m1[b, :nw].cpu().numpy(), mo1)
        ls = {"K": np64(s["K"]), "V": np64(s["V"]), "Z": st(zo), "M": mo}
        ls1 = {"K": np64(s["K1"]), "V": np64(s["V1"]), "Z": st(zo1), "M": mo1}
        if nv:
            ls["codes"], ls["scales"] = O.residual_quantize(Hb, ls["Z"], mo, w.resid)
            ls1["codes"], ls1["scales"] = O.residual_quantize(np64(s["H1"]), ls1["Z"], mo1, w.resid)
            assert np.array_equal(codes[b, :nw].cpu().numpy(), ls["codes"]), f"entry {w.resid} codes differ"
            assert np.array_equal(scales[b, :nw, :sb].cpu().numpy(), ls["scales"])
        else:
            ls["H"] = Hb
            ls1["H"] = np64(s["H1"])
        # first drift reference: proxy logits of the entry centroids over the proxy keys (oracle ->
        # device); the other key positions hold seeded noise that the drift must not read
        zq = O.project(ls["Z"], Wo["wq"], cfg.eps, st).reshape(K, hq, dh)
        keys = O.proxy_keys(cfg, blk_start)
        _, pl = O.attention(zq, ls["K"][keys], ls["V"][keys], hq, hkv)
        ls["P"] = O.round_f32(np64(synth.tensor(w, (b, 41), (K, hq, n), 3.0, 0, "cpu", "f32")))
        ls["P"][..., keys] = O.round_f32(pl)
        plog[b] = torch.tensor(ls["P"], dtype=torch.float32)
        # keep both sides on identical state: device gets the oracle's centroids
        z[b] = to_dev(ls["Z"], w.dtype)
        z1[b] = to_dev(ls1["Z"], w.dtype)
        OL.append(ls)
        OL1.append(ls1)
    log("[layer-parity] entry ok")

    # ---- 2. window update with an incoming packet
    u_rows = dev.zeros(batch, WM, d)
    u_idx = torch.zeros(batch, WM, dtype=torch.int32, device="cuda")
    u_cnt = torch.zeros(batch, dtype=torch.int32, device="cuda")
    for b, s in enumerate(S):
        c = len(s["u_idx"])
        u_rows[b, :c] = s["u_rows"]
        u_idx[b, :c] = torch.tensor(s["u_idx"])
        u_cnt[b] = c
    pin = packet(u_rows, u_idx, u_cnt)
    B.polestar_cluster(dev.h, B.CLUSTER_UPDATE, Ls0, blk_start, pin, None, None, None, dev.ws, dev.ws_bytes)
    torch.cuda.synchronize()
    CU = []
    for b, s in enumerate(S):
        cu = O.cluster_update(OL[b], cfg, np64(s["u_rows"]), s["u_idx"])
        CU.append(cu)
        assert_stored(np64(z[b]), OL[b]["Z"], w.dtype, "updated centroids")
        if nv:
            assert np.array_equal(codes[b, :nw].cpu().numpy(), OL[b]["codes"]), "re-quantised codes differ"
            assert np.array_equal(scales[b, :nw, :sb].cpu().numpy(), OL[b]["scales"])
        else:
            assert np.array_equal(np64(win[b, :nw]), OL[b]["H"]), "patched window rows differ"
        z[b] = to_dev(OL[b]["Z"], w.dtype)
    log("[layer-parity] window update ok")

    # ---- 3. drift
    chk_qkv = torch.zeros(batch, dev.win_max + Bk + K, (hq + 2 * hkv) * dh, dtype=torch.float32, device="cuda")
    chk_att = torch.zeros(batch, Bk + WM, hq * dh, dtype=torch.float32, device="cuda")
    chk_hp = torch.zeros(batch, Bk + WM, d, dtype=torch.float32, device="cuda")
    chk_out = torch.zeros(batch, Bk + WM, d, dtype=torch.float32, device="cuda")
    chk_kv = torch.zeros(batch, WM, 2 * hkv * dh, dtype=torch.float32, device="cuda")
    chk = B.Check(qkv=chk_qkv.data_ptr(), attn_out=chk_att.data_ptr(), hp=chk_hp.data_ptr(), out=chk_out.data_ptr(),
                  kv_next=chk_kv.data_ptr())
    B.polestar_set_check(dev.h, chk)
    h_act = torch.stack([s["h_act"] for s in S]).contiguous()
    act_logits = torch.stack([s["act_prev"] for s in S]).contiguous()
    D = torch.zeros(batch, K, dtype=torch.float32, device="cuda")
    topk = torch.zeros(batch, w.top_k, dtype=torch.int32, device="cuda")
    sel_idx = torch.zeros(batch, WM, dtype=torch.int32, device="cuda")
    sel_cnt = torch.zeros(batch, dtype=torch.int32, device="cuda")
    delta = torch.zeros(batch, Bk, dtype=torch.float32, device="cuda")
    sel = packet(None, sel_idx, sel_cnt)
    kc_before = kc.clone()
    B.polestar_drift(dev.h, B.DRIFT_REFRESH, Ls0, blk_start, h_act, pin, D, topk, sel, act_logits, delta, dev.ws,
                     dev.ws_bytes)
    torch.cuda.synchronize()
    DR, ALLOW = [], []
    nq, nkv = hq * dh, hkv * dh
    for b, s in enumerate(S):
        ha = np64(s["h_act"])
        P_before = np.array(OL[b]["P"], copy=True)
        dr = O.drift_layer(OL[b], Wo, cfg, blk_start, ha, CU[b]["h"], CU[b]["patched"], True,
                           commit_prev=np64(s["act_prev"]))
        DR.append(dr)
        toks = np.concatenate([ha, CU[b]["h"]], 0)
        wqkv = np.concatenate([Wo["wq"], Wo["wk"], Wo["wv"]], 0)
        proj = np.concatenate([O.project(toks, wqkv, cfg.eps, st), O.project(OL[b]["Z"], wqkv, cfg.eps, st)], 0)
        # admissible deviations (oracle values only): the projection inputs round(RMSNorm(x)) and the
        # K/V rows this call stores, which its attention then reads
        al = FL.drift_call_allow(O, cfg, Wo, blk_start, ha, CU[b]["h"], CU[b]["patched"], OL[b]["Z"],
                                 OL[b]["K"], OL[b]["V"], dr["proxy_q"], dr["proxy_keys"], P_before,
                                 act_prev=np64(s["act_prev"]))
        assert_close(chk_qkv[b, : Bk + nw + K].cpu().numpy(), proj, "QKV projections", dtype=w.dtype,
                     allow=al["qkv"])
        pk = dr["proxy_keys"]
        ALLOW.append(al)
        # caches: active rows and patched rows rewritten, every other row bit-identical
        assert_stored(np64(kc[b]).reshape(n, -1), OL[b]["K"].reshape(n, -1), w.dtype, "K cache")
        assert_stored(np64(vc[b].permute(2, 0, 1)).reshape(n, -1), OL[b]["V"].reshape(n, -1), w.dtype, "V cache")
        untouched = np.setdiff1d(np.arange(n), np.concatenate([np.arange(blk_start, blk_start + Bk),
                                                              wpos[s["u_idx"]]]))
        assert torch.equal(kc[b, untouched], kc_before[b, untouched])
        assert_close(chk_att[b, : Bk + nw].cpu().numpy(), dr["o"], "attention outputs", dtype=w.dtype, allow=al["o"])
        assert_close(plog[b].cpu().numpy()[..., pk], dr["proxy_logits"], "proxy logits", dtype=w.dtype,
                     allow=al["proxy_logits"], floor=LOGIT_FLOOR)
        outside = np.setdiff1d(np.arange(n), pk)
        assert np.array_equal(plog[b].cpu().numpy()[..., outside], OL[b]["P"][..., outside]), \
            "proxy logits outside the proxy keys were written"
        assert_close(act_logits[b].cpu().numpy(), dr["act_logits"], "active logits", dtype=w.dtype,
                     allow=al["act_logits"], floor=LOGIT_FLOOR)
        assert_close(delta[b].cpu().numpy(), dr["delta"], "active drift delta", allow=al["delta"])
        Dg = D[b].cpu().numpy()
        assert_close(Dg, dr["D"], "cluster drift D", allow=al["D"])
        tg = topk[b].cpu().numpy()
        assert check_topk(tg, Dg, dr["D"], dr["topk"], w.top_k, keff, f"seq {b}", al["D"]), "top-k near-tie"
        cnt = int(sel_cnt[b])
        assert np.array_equal(sel_idx[b, :cnt].cpu().numpy(), dr["S"]), "selected rows S differ"
        log(f"[layer-parity] seq {b}: D={np.round(Dg, 5).tolist()} topk={tg.tolist()} nS={cnt}")
    log("[layer-parity] drift ok")

    # ---- 4. sparse forward + next-layer K/V
    h_out = dev.zeros(batch, Bk, d)
    u_new = dev.zeros(batch, WM, d)
    B.polestar_refresh(dev.h, Ls0, blk_start, h_act, sel, wkv1, kc1, vc1, h_out, u_new, dev.ws, dev.ws_bytes)
    torch.cuda.synchronize()
    RF = []
    for b, s in enumerate(S):
        Sb = DR[b]["S"]
        rf = O.refresh_layer(Wo, cfg, np64(s["h_act"]), CU[b]["h"], DR[b]["o"], Sb)
        RF.append(rf)
        rows = Bk + len(Sb)
        out_pre = chk_out[b, :rows].cpu().numpy()
        ar = FL.refresh_call_allow(O, cfg, Wo, rf, ALLOW[b]["o"], Sb, np.concatenate([wk1, wv1], 0))
        dhp, dout = ar["hp"], ar["out"]
        assert_close(chk_hp[b, :rows].cpu().numpy(), rf["hp"], "h' = h + o W_O", dtype=w.dtype, allow=dhp)
        assert_close(out_pre, rf["out_pre"], "layer outputs", dtype=w.dtype, allow=dout)
        assert_rounded(np64(h_out[b]), out_pre[:Bk], w.dtype, "active outputs")
        assert_rounded(np64(u_new[b, : len(Sb)]), out_pre[Bk:], w.dtype, "update packet U")
        assert_stored(np64(h_out[b]), rf["h_act_out"], w.dtype, "active outputs")
        assert_stored(np64(u_new[b, : len(Sb)]), rf["U"], w.dtype, "update packet U")
        # next layer's K/V: projections of round(RMSNorm(U)), each side from its own stored U
        k1, v1 = O.kv_rows(rf["U"], wk1, wv1, cfg)
        pre = np.concatenate([O.project(rf["U"], wk1, cfg.eps, st), O.project(rf["U"], wv1, cfg.eps, st)], 1)
        kv_pre = chk_kv[b, : len(Sb)].cpu().numpy()
        assert_close(kv_pre, pre, "next-layer K/V projections", dtype=w.dtype, allow=ar["kv"])
        pos = wpos[Sb]
        nkv = hkv * dh
        assert_rounded(np64(kc1[b, pos]).reshape(len(pos), -1), kv_pre[:, :nkv], w.dtype, "next-layer K rows")
        assert_rounded(np64(vc1[b].permute(2, 0, 1)[pos]).reshape(len(pos), -1), kv_pre[:, nkv:], w.dtype,
                       "next-layer V rows")
        log(f"    next-layer K/V rows vs the oracle's stored rows: max row err "
            f"{row_err(np64(kc1[b, pos]).reshape(len(pos), -1), k1.reshape(len(pos), -1)).max():.2e} (K), "
            f"{row_err(np64(vc1[b].permute(2, 0, 1)[pos]).reshape(len(pos), -1), v1.reshape(len(pos), -1)).max():.2e} (V)")
        others = np.setdiff1d(np.arange(n), pos)
        assert torch.equal(kc1[b, others], S[b]["K1"][others])
    log("[layer-parity] refresh ok")

    # ---- 5. layer l+1 takes the packet: window rows patched, centroids refreshed
    pout = packet(u_new, sel_idx, sel_cnt)
    B.polestar_cluster(dev.h, B.CLUSTER_UPDATE, Ls1, blk_start, pout, None, None, None, dev.ws, dev.ws_bytes)
    torch.cuda.synchronize()
    for b in range(batch):
        O.cluster_update(OL1[b], cfg, RF[b]["U"], DR[b]["S"])
        assert_stored(np64(z1[b]), OL1[b]["Z"], w.dtype, "layer l+1 centroids")
        if not nv:
            assert_stored(np64(win1[b, :nw]), OL1[b]["H"], w.dtype, "layer l+1 window rows")
    B.polestar_set_check(dev.h, None)
    dev.close()
    log(f"[layer-parity] case={case} passed")


def test_drift_is_deterministic():
    """Identical inputs give bit-identical outputs across two runs."""
    w = synth.WORKLOADS[2]
    dev = Dev(w, batch=1, vocab=0)
    n, d, hq, hkv, dh, Bk = w.n_pos, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.block
    wpos = O.window_positions(w.prompt, n, Bk, w.win_prefix, w.win_suffix)
    nw, WM, K = len(wpos), dev.win_max, w.n_clusters
    P0 = packed_layer(dev, weights(w, 0))
    s = _state(w, dev, 0, nw)
    outs = []
    for rep in range(2):
        kc, vc = s["K"][None].clone(), s["V"].permute(1, 2, 0)[None].contiguous()
        win = dev.zeros(1, WM, d)
        win[0, :nw] = s["H"]
        z, m = dev.zeros(1, K, d), torch.zeros(1, WM, dtype=torch.int32, device="cuda")
        plog = synth.tensor(w, (0, 40), (1, K, hq, n), 1.0, 0, "cuda", "f32")
        init = torch.tensor(s["init"], dtype=torch.int32, device="cuda")[None]
        Ls = layer_struct(dict(P0, k_cache=kc, v_cache=vc, win_h=win, win_z=z, win_m=m, proxy_logits=plog))
        B.polestar_cluster(dev.h, B.CLUSTER_ENTRY, Ls, w.prompt, None, init, win, None, dev.ws, dev.ws_bytes)
        B.polestar_cluster(dev.h, B.CLUSTER_UPDATE, Ls, w.prompt, None, None, None, None, dev.ws, dev.ws_bytes)
        D = torch.zeros(1, K, dtype=torch.float32, device="cuda")
        sel_idx = torch.zeros(1, WM, dtype=torch.int32, device="cuda")
        sel_cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
        sel = packet(None, sel_idx, sel_cnt)
        h_act = s["h_act"][None].contiguous()
        B.polestar_drift(dev.h, B.DRIFT_REFRESH, Ls, w.prompt, h_act, None, D, None, sel, None, None, dev.ws,
                         dev.ws_bytes)
        h_out, u_new = dev.zeros(1, Bk, d), dev.zeros(1, WM, d)
        B.polestar_refresh(dev.h, Ls, w.prompt, h_act, sel, None, None, None, h_out, u_new, dev.ws, dev.ws_bytes)
        torch.cuda.synchronize()
        outs.append((D.clone(), sel_idx.clone(), h_out.clone(), u_new.clone(), kc.clone(), plog.clone(), z.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    dev.close()
