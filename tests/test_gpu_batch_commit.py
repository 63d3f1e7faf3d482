"""The batched refresh with the commit at its full size: 16 LLaDA-shaped sequences of
prompt 512 + gen 256, 32 layers, window residuals stored as NVFP4 and dequantised in
the refresh, the last layer's LM head over 126464 ids and the commit rule, in the
launch configuration the benchmark times (the stack's per-layer calls, then
polestar_commit).  The GPU runs every sequence; two of them (the first and the
last) are checked against the oracle along trigger-driven steps.

Per call, as in the trajectory tests: the rows passed from one layer to the next
(active rows, update packet) and the state carried to the next step are the
oracle's stored values for the checked sequences on both sides; S bit-exact;
drift D within 2e-3 elementwise plus the oracle-derived allowance of admissible
tie roundings; stored tensors within the stored-value bounds; residual codes
bit-exact.  The commit of every step: confidences within 2e-3 of the oracle's,
argmax ids exact, and commit masks from the oracle's own confidences and drift,
different only at reported near-threshold rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from drift_driven_sparse_amd.stack import RefreshStack
from oracle import polestar_oracle as O
from tests import flips as FL
from tests.harness import assert_close, assert_stored, check_topk, log, np64, to_dev
from tests.test_gpu_commit import C_TOL, _check_masks, _lm_logits

pytestmark = pytest.mark.gpu

CHECKED = (0, 15)


@pytest.mark.timeout(900)
def test_batch16_nvfp4_stack_with_commit():
    w = synth.WORKLOADS[5]
    n_layers, steps, bt = w.n_layers, 3, w.batch
    n, d, hq, hkv, dh, Bk, K = w.n_pos, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.block, w.n_clusters
    blk = w.prompt
    cfg = O.Cfg.from_workload(w)
    st_ = cfg.st
    wpos = O.window_positions(blk, n, Bk, w.win_prefix, w.win_suffix)
    nw = len(wpos)
    n_pre = int(np.sum(wpos < blk))
    mask_id = w.vocab - 1
    log(f"[batch-commit] {w.name}: {n_layers} layers, batch {bt}, n {n}, vocab {w.vocab}, checked {CHECKED}")
    dims = B.Dims(d=d, n_heads=hq, n_kv_heads=hkv, head_dim=dh, ffn=w.ffn, n_pos=n, batch=bt, block=Bk,
                  win_prefix=w.win_prefix, win_suffix=w.win_suffix, n_clusters=K, top_k=w.top_k, vocab=w.vocab,
                  dtype=B.BF16, resid_fmt=B.RESID_NVFP4)
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist,
                      mask_id=mask_id, kmeans_iters=w.kmeans_iters)
    st = RefreshStack(dims, params, n_layers)
    try:
        # ---- seeded block-entry state of every sequence; the oracle's for the checked ones
        OL = [dict() for _ in range(n_layers)]
        for l in range(n_layers):
            st.set_layer_weights(l, synth.layer_weights(w, l, device="cuda"))
            L = st.layers[l]
            L["k_cache"].copy_(synth.tensor(w, (l, 10), L["k_cache"].shape, 1.0, 0, "cuda", "bf16"))
            L["v_cache"].copy_(synth.tensor(w, (l, 11), L["v_cache"].shape, 1.0, 0, "cuda", "bf16"))
            L["proxy_logits"].copy_(synth.tensor(w, (l, 13), L["proxy_logits"].shape, 3.0, 0, "cuda", "f32"))
            rows = synth.tensor(w, (l, 12), (bt, st.win_max, d), 1.0, 0, "cuda", "bf16")
            init = torch.stack([torch.tensor(synth.kmeans_init(w, nw, l, 0, 0, b), dtype=torch.int32)
                                for b in range(bt)]).cuda()
            B.polestar_cluster(st.h, B.CLUSTER_ENTRY, st.struct(l), blk, None, init, rows, None, st.ws, st.ws_bytes)
            torch.cuda.synchronize()
            Wq = np64(synth.weight(w, l, "wq", device="cuda"))
            Kg = synth.tensor(w, (l, 10), L["k_cache"].shape, 1.0, 0, "cuda", "bf16")   # the generator's values
            Vg = synth.tensor(w, (l, 11), L["v_cache"].shape, 1.0, 0, "cuda", "bf16")
            for b in CHECKED:
                H = np.zeros((n, d))
                H[wpos] = np64(rows[b, :nw])
                ls = O.block_entry_layer_state(H, np64(Kg[b]), np64(Vg[b].permute(2, 0, 1)), Wq, cfg, blk,
                                               synth.kmeans_init(w, nw, l, 0, 0, b))
                assert np.array_equal(L["win_m"][b, :nw].cpu().numpy(), ls["M"]), f"layer {l} seq {b}: labels"
                assert np.array_equal(L["win_codes"][b, :nw].cpu().numpy(), ls["codes"]), f"layer {l} seq {b}: codes"
                L["win_z"][b] = to_dev(ls["Z"], "bf16")
                L["proxy_logits"][b] = torch.tensor(ls["P"], dtype=torch.float32)
                OL[l][b] = ls
        st.set_lm_head(synth.weight(w, 0, "wlm", device="cuda"))
        act_prev = {b: O.round_f32(np64(synth.tensor(w, (61, b), (Bk, hq, n), 1.0, 0, "cpu", "f32"))) for b in CHECKED}
        for b in CHECKED:
            st.act_logits[b] = torch.tensor(act_prev[b], dtype=torch.float32)
        hist = {b: (np.zeros((Bk, max(w.hist, 1)), np.float32), np.zeros(Bk, np.int32)) for b in CHECKED}
        hist_allow = {b: [] for b in CHECKED}   # allowances of the drift values in each history
        ha_vals = {b: [] for b in CHECKED}      # and the values
        torch.cuda.synchronize()
        log("[batch-commit] entry state ready")

        sched = synth.unmask_schedule(w, steps=steps)
        x0 = synth.tensor(w, (60,), (bt, Bk, d), 1.0, 0, "cuda", "bf16")
        decoded, kinds = 0, []
        for t in range(steps):
            _, offs = sched[t]
            for b in range(bt):
                for o in offs:
                    x0[b, o] = (x0[b, o].float() + synth.unmask_noise(w, t, blk + o, 0, b, "cuda")).to(torch.bfloat16)
            decoded += len(offs)
            refresh = B.polestar_should_refresh(decoded, w.tau_upd)
            if refresh:
                decoded = 0
            kinds.append(refresh)
            st.h_act[0].copy_(x0)
            x = {b: np64(x0[b]) for b in CHECKED}
            cur, pk = 0, 0
            u_in, U_prev, S_prev = None, {b: None for b in CHECKED}, {b: None for b in CHECKED}
            for l in range(n_layers):
                last = l == n_layers - 1
                tag = f"step {t} layer {l} ({'refresh' if refresh else 'active only'})"
                Ls = st.struct(l)
                if refresh:
                    B.polestar_cluster(st.h, B.CLUSTER_UPDATE, Ls, blk, u_in, None, None, None, st.ws, st.ws_bytes)
                sel = st.packets[pk]
                B.polestar_drift(st.h, B.DRIFT_REFRESH if refresh else B.DRIFT_ACTIVE_ONLY, Ls, blk, st.h_act[cur],
                                 u_in, st.D, st.topk, sel, st.act_logits if last else None,
                                 st.delta if last else None, st.ws, st.ws_bytes)
                torch.cuda.synchronize()
                W = {k: np64(v) for k, v in synth.layer_weights(w, l, device="cuda").items()}
                DR = {}
                for b in CHECKED:
                    ls = OL[l][b]
                    if refresh:
                        cu = O.cluster_update(ls, cfg, U_prev[b], S_prev[b])
                        h_win, patched = cu["h"], cu["patched"]
                        assert np.array_equal(st.layers[l]["win_codes"][b, :nw].cpu().numpy(), ls["codes"]), \
                            f"{tag} seq {b}: re-quantised codes"
                    else:
                        h_win, patched = O.window_rows_now(ls, cfg), None
                    P_before = ls["P"].copy()
                    a_prev = act_prev[b] if last else None
                    dr = O.drift_layer(ls, W, cfg, blk, x[b], h_win, patched, refresh, commit_prev=a_prev)
                    al = FL.drift_call_allow(O, cfg, W, blk, x[b], h_win, patched, ls["Z"], ls["K"], ls["V"],
                                             dr.get("proxy_q"), dr.get("proxy_keys"), P_before, act_prev=a_prev,
                                             refresh=refresh)
                    DR[b] = (dr, h_win, al)
                    if last:
                        assert_close(st.delta[b].cpu().numpy(), dr["delta"], f"{tag} seq {b}: active drift delta",
                                     allow=al["delta"])
                    if refresh:
                        Dg = st.D[b].cpu().numpy()
                        assert_close(Dg, dr["D"], f"{tag} seq {b}: cluster drift D", allow=al["D"])
                        if not check_topk(st.topk[b].cpu().numpy(), Dg, dr["D"], dr["topk"], w.top_k, min(K, nw),
                                          f"{tag} seq {b}", D_allow=al["D"]):
                            st.pk_idx[pk][b, : len(dr["S"])] = torch.tensor(dr["S"], dtype=torch.int32)
                            st.pk_cnt[pk][b] = len(dr["S"])
                        cnt = int(st.pk_cnt[pk][b])
                        assert np.array_equal(st.pk_idx[pk][b, :cnt].cpu().numpy(), dr["S"]), f"{tag} seq {b}: S"
                    if last:
                        act_prev[b] = dr["act_logits"]
                B.polestar_refresh(st.h, Ls, blk, st.h_act[cur], sel, None, None, None, st.h_act[1 - cur],
                                   st.pk_rows[pk], st.ws, st.ws_bytes)
                torch.cuda.synchronize()
                for b in CHECKED:
                    dr, h_win, al = DR[b]
                    S = dr["S"] if refresh else np.zeros(0, dtype=np.int64)
                    rf = O.refresh_layer(W, cfg, x[b], h_win, dr["o"], S)
                    if refresh:
                        assert_stored(np64(st.pk_rows[pk][b, : len(S)]), rf["U"], "bf16", f"{tag} seq {b}: U")
                        st.pk_rows[pk][b, : len(S)] = to_dev(rf["U"], "bf16")
                        U_prev[b], S_prev[b] = rf["U"], S
                    assert_stored(np64(st.h_act[1 - cur][b]), rf["h_act_out"], "bf16", f"{tag} seq {b}: active outputs")
                    st.h_act[1 - cur][b] = to_dev(rf["h_act_out"], "bf16")
                    x[b] = rf["h_act_out"]
                    if last:
                        DR[b] = (dr, h_win, rf, al)
                del W
                u_in = sel if refresh else None
                cur, pk = 1 - cur, 1 - pk
            st.last_packet = 1 - pk
            # ---- the commit of this step
            st.commit(blk, st.h_act[cur])
            torch.cuda.synchronize()
            for b in CHECKED:
                dr, _, rf, al = DR[b]
                S = dr["S"] if refresh else np.zeros(0, dtype=np.int64)
                suf = [i for i, s in enumerate(S) if s >= n_pre]
                rows = np.concatenate([rf["h_act_out"], rf["U"][suf]], 0) if refresh else rf["h_act_out"]
                c, yhat = O.confidence_from_logits(_lm_logits(w, rows, w.rms_eps), mask_id)
                ca = c[:Bk]
                cg = st.conf_active[b].cpu().numpy()
                assert np.max(np.abs(cg - ca) / ca) <= C_TOL, f"step {t} seq {b}: active confidences"
                assert np.array_equal(st.yhat_active[b].cpu().numpy(), yhat[:Bk]), f"step {t} seq {b}: argmax ids"
                hv, hc = hist[b]
                com, sp, _, hv, hc = O.commit_decide(dr["delta"], ca.astype(np.float32), np.ones(Bk, bool), hv, hc,
                                                     w.hist, w.alpha, w.tau_s)
                hist[b] = (hv, hc)
                # spike = delta - mean of the history: its allowance is delta's plus the mean of the
                # history's allowances, and each side's delta values differ within 2e-3
                ha = hist_allow[b]
                mean_al = np.mean(ha, axis=0) if ha else np.zeros(Bk)
                mean_tol = 2e-3 * np.mean([np.abs(v) for v in ha_vals[b]], axis=0) if ha_vals[b] else np.zeros(Bk)
                spg = st.spike[b].cpu().numpy()
                sp_allow = al["delta"] + mean_al + mean_tol
                assert_close(spg, sp, f"step {t} seq {b}: drift spikes", allow=sp_allow)
                ha.append(al["delta"])
                ha_vals[b].append(dr["delta"])
                if w.hist > 0:
                    del ha[:-w.hist]
                    del ha_vals[b][:-w.hist]
                sp_tol = 2e-3 * np.maximum(np.abs(sp), 1e-3 * np.abs(sp).max()) + sp_allow
                _check_masks(st.commit_active[b].cpu().numpy(), com, ca, w.tau_s, f"step {t} seq {b} active", sp,
                             w.alpha, spike_tol=sp_tol)
                conf_suf = np.zeros(w.win_suffix)
                for j, i in enumerate(suf):
                    conf_suf[int(S[i]) - n_pre] = c[Bk + j]
                gs = st.conf_suffix[b].cpu().numpy()
                assert np.all(np.abs(gs - conf_suf) <= C_TOL * np.maximum(conf_suf, 1e-30)), \
                    f"step {t} seq {b}: suffix confidences"
                want = O.suffix_commit(conf_suf.astype(np.float32), conf_suf > 0, w.tau_suf)
                _check_masks(st.commit_suffix[b].cpu().numpy(), want, conf_suf, w.tau_suf, f"step {t} seq {b} suffix")
                log(f"    step {t} seq {b}: confidences max {ca.max():.4f}, {int(com.sum())} active commits, "
                    f"{len(suf)} suffix rows")
            # the carried state: compared, then both sides continue from the oracle's copy
            for l in range(n_layers):
                L = st.layers[l]
                for b in CHECKED:
                    ls = OL[l][b]
                    assert_stored(np64(L["k_cache"][b]).reshape(n, -1), ls["K"].reshape(n, -1), "bf16",
                                  f"step {t} layer {l} seq {b}: K")
                    assert_stored(np64(L["win_z"][b]), ls["Z"], "bf16", f"step {t} layer {l} seq {b}: centroids")
                    L["k_cache"][b] = to_dev(ls["K"], "bf16")
                    L["v_cache"][b] = to_dev(ls["V"], "bf16").permute(1, 2, 0)
                    L["win_z"][b] = to_dev(ls["Z"], "bf16")
                    L["proxy_logits"][b] = torch.tensor(ls["P"], dtype=torch.float32)
            for b in CHECKED:
                st.act_logits[b] = torch.tensor(act_prev[b], dtype=torch.float32)
            log(f"[batch-commit] step {t} ok ({'refresh' if refresh else 'active only'}, {len(offs)} decoded)")
        assert any(kinds), "the trigger gave no refresh step"
        # every sequence: finite outputs and a sane commit
        assert torch.isfinite(st.conf_active).all() and (st.conf_active > 0).all() and (st.conf_active <= 1).all()
    finally:
        st.close()
    log("[batch-commit] passed")
