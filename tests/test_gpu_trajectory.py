"""GPU parity over a free-running trajectory: several denoising steps of a small
layer stack, refresh steps (window update, drift, top-k, sparse forward,
update packet to the next layer) interleaved with steps without a refresh
(active rows only), and the last layer's active drift for the commit rule.

Both sides start from the oracle's block-entry state (dense forward of all
positions, k-means of the window rows, proxy logits).  Each step feeds the
same seeded layer-0 active rows to both; every later value is each side's own.
Per step and layer the top-k clusters and the selected rows must match; every
floating-point tensor (drift values, active outputs, update packets, logits and
the state below) must stay within 2e-3 normwise per tensor, and for bf16
storage within one bf16 ulp normwise per row and a few ulps per element, since
each side continues from its own stored values.  At the end of each step the state each side
carries into the next one (K/V caches, window rows or NVFP4 codes, centroids,
proxy logits, active logits) is compared, then the oracle's copy is written
back to the device so that storage-rounding differences of one step do not
compound into the next.  A top-k selection whose oracle margin is below 1e-3
ends the comparison (both selections are then admissible).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O
from tests.harness import (Dev, assert_traj, check_topk, layer_struct, log, np64, packed_layer,
                           packet, to_dev, weights)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, layers, steps)
    "tiny_fp32_2layers": (synth.WORKLOADS[1], 2, 8),
    "tiny_bf16_2layers": (synth.shrink(synth.WORKLOADS[1], dtype="bf16"), 2, 8),
    "tiny_bf16_nvfp4_2layers": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", resid="nvfp4"), 2, 6),
}


def _refresh_at(t: int) -> bool:
    return t % 3 != 2


@pytest.mark.parametrize("case", list(CASES))
def test_trajectory_parity(case):
    w, n_layers, steps = CASES[case]
    log(f"[trajectory] case={case} d={w.d} n={w.n_pos} layers={n_layers} steps={steps} dtype={w.dtype} "
        f"resid={w.resid}")
    torch.manual_seed(0)
    dev = Dev(w, batch=1, vocab=0)
    cfg = O.Cfg.from_workload(w, top_k=w.top_k)
    st = cfg.st
    n, d, hq, hkv, dh, Bk, K = w.n_pos, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.block, w.n_clusters
    blk_start = w.prompt
    wpos = O.window_positions(blk_start, n, Bk, w.win_prefix, w.win_suffix)
    nw, WM = len(wpos), dev.win_max
    keff = min(K, nw)
    nv = w.resid == "nvfp4"
    try:
        # ---- weights and the block-entry state (oracle)
        Wd = [weights(w, l) for l in range(n_layers)]
        Wo = [{k: np64(v) for k, v in W.items()} for W in Wd]
        P = [packed_layer(dev, W) for W in Wd]
        del Wd
        h0 = st(np64(synth.embeddings(w)))
        Hs, Ks, Vs, last_logits = O.full_forward(h0, Wo, cfg)
        OL, L, Ls = [], [], []
        for l in range(n_layers):
            init = synth.kmeans_init(w, nw, l, 0)
            ls = O.block_entry_layer_state(Hs[l], Ks[l], Vs[l], Wo[l]["wq"], cfg, blk_start, init)
            OL.append(ls)
            Ld = dict(P[l])
            Ld["k_cache"] = to_dev(ls["K"], w.dtype)[None].contiguous()
            Ld["v_cache"] = to_dev(ls["V"], w.dtype).permute(1, 2, 0)[None].contiguous()
            Ld["win_z"] = to_dev(ls["Z"], w.dtype)[None].contiguous()
            m = torch.zeros(1, WM, dtype=torch.int32, device="cuda")
            m[0, :nw] = torch.tensor(ls["M"], dtype=torch.int32)
            Ld["win_m"] = m
            Ld["proxy_logits"] = torch.tensor(ls["P"], dtype=torch.float32, device="cuda")[None].contiguous()
            if nv:
                c = torch.zeros(1, WM, d // 2, dtype=torch.uint8, device="cuda")
                s = torch.zeros(1, WM, d // 16, dtype=torch.uint8, device="cuda")
                c[0, :nw] = torch.tensor(ls["codes"])
                s[0, :nw] = torch.tensor(ls["scales"])
                Ld["win_codes"], Ld["win_scales"] = c, s
            else:
                hw = dev.zeros(1, WM, d)
                hw[0, :nw] = to_dev(ls["H"], w.dtype)
                Ld["win_h"] = hw
            L.append(Ld)
            Ls.append(layer_struct(Ld))
        # active drift reference: the entry forward's last-layer logits of the active rows
        act_prev = O.round_f32(last_logits[blk_start: blk_start + Bk])
        act_logits = torch.tensor(act_prev, dtype=torch.float32, device="cuda")[None].contiguous()
        log("[trajectory] entry state ready")

        # ---- device step buffers
        h_act = [dev.zeros(1, Bk, d) for _ in range(2)]
        pk_rows = [dev.zeros(1, WM, d) for _ in range(2)]
        pk_idx = [torch.zeros(1, WM, dtype=torch.int32, device="cuda") for _ in range(2)]
        pk_cnt = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]
        pks = [packet(pk_rows[i], pk_idx[i], pk_cnt[i]) for i in range(2)]
        D = torch.zeros(1, K, dtype=torch.float32, device="cuda")
        topk = torch.zeros(1, w.top_k, dtype=torch.int32, device="cuda")
        delta = torch.zeros(1, Bk, dtype=torch.float32, device="cuda")

        for t in range(steps):
            refresh = _refresh_at(t)
            # layer-0 active rows: the entry input plus the step's unmasking noise
            noise = np64(synth.tensor(w, (77, t), (Bk, d), np.sqrt(w.noise_var)))
            x = st(h0[blk_start: blk_start + Bk] + noise)
            h_act[0][0] = to_dev(x, w.dtype)
            cur, pk = 0, 0
            u_in, U_prev, S_prev = None, None, None
            for l in range(n_layers):
                last = l == n_layers - 1
                # device
                if refresh:
                    B.polestar_cluster(dev.h, B.CLUSTER_UPDATE, Ls[l], blk_start, u_in, None, None, None, dev.ws,
                                       dev.ws_bytes)
                sel = pks[pk]
                B.polestar_drift(dev.h, B.DRIFT_REFRESH if refresh else B.DRIFT_ACTIVE_ONLY, Ls[l], blk_start,
                                 h_act[cur], u_in, D, topk, sel, act_logits if last else None,
                                 delta if last else None, dev.ws, dev.ws_bytes)
                B.polestar_refresh(dev.h, Ls[l], blk_start, h_act[cur], sel, None, None, None, h_act[1 - cur],
                                   pk_rows[pk], dev.ws, dev.ws_bytes)
                torch.cuda.synchronize()
                # oracle
                ls = OL[l]
                if refresh:
                    cu = O.cluster_update(ls, cfg, U_prev, S_prev)
                    h_win, patched = cu["h"], cu["patched"]
                else:
                    h_win, patched = O.window_rows_now(ls, cfg), None
                dr = O.drift_layer(ls, Wo[l], cfg, blk_start, x, h_win, patched, refresh,
                                   commit_prev=act_prev if last else None)
                S = dr["S"] if refresh else np.zeros(0, dtype=np.int64)
                rf = O.refresh_layer(Wo[l], cfg, x, h_win, dr["o"], S)
                tag = f"step {t} layer {l} ({'refresh' if refresh else 'active only'})"
                if refresh:
                    Dg = D[0].cpu().numpy()
                    assert_traj(Dg, dr["D"], w.dtype, f"{tag}: cluster drift D")
                    if not check_topk(topk[0].cpu().numpy(), Dg, dr["D"], dr["topk"], w.top_k, keff, tag):
                        log(f"[trajectory] {tag}: trajectories part here")
                        return
                    cnt = int(pk_cnt[pk][0])
                    assert np.array_equal(pk_idx[pk][0, :cnt].cpu().numpy(), dr["S"]), f"{tag}: rows S differ"
                    assert_traj(np64(pk_rows[pk][0, :cnt]), rf["U"], w.dtype, f"{tag}: update packet U")
                else:
                    assert int(pk_cnt[pk][0]) == 0
                assert_traj(np64(h_act[1 - cur][0]), rf["h_act_out"], w.dtype, f"{tag}: active outputs")
                if last:
                    assert_traj(delta[0].cpu().numpy(), dr["delta"], w.dtype, f"{tag}: active drift delta")
                    act_prev = dr["act_logits"]
                # both sides continue from their own values
                x = rf["h_act_out"]
                if refresh:
                    u_in, U_prev, S_prev = pks[pk], rf["U"], dr["S"]
                cur, pk = 1 - cur, 1 - pk
            # carried state: compare, then continue from the oracle's copy on both sides
            for l in range(n_layers):
                ls, Ld, tag = OL[l], L[l], f"step {t} layer {l} state"
                assert_traj(np64(Ld["k_cache"][0]).reshape(n, -1), ls["K"].reshape(n, -1), w.dtype, f"{tag}: K")
                assert_traj(np64(Ld["v_cache"][0].permute(2, 0, 1)).reshape(n, -1), ls["V"].reshape(n, -1),
                              w.dtype, f"{tag}: V")
                assert_traj(np64(Ld["win_z"][0]), ls["Z"], w.dtype, f"{tag}: centroids")
                assert np.array_equal(Ld["win_m"][0, :nw].cpu().numpy(), ls["M"]), f"{tag}: labels changed"
                assert_traj(Ld["proxy_logits"][0].cpu().numpy(), ls["P"], w.dtype, f"{tag}: proxy logits")
                if nv:
                    frac = float(np.mean(Ld["win_codes"][0, :nw].cpu().numpy() != ls["codes"]))
                    log(f"    {tag}: {frac:.3%} NVFP4 code bytes differ")
                    assert frac < 0.05, f"{tag}: NVFP4 codes differ in {frac:.2%} of bytes"
                    Ld["win_codes"][0, :nw] = torch.tensor(ls["codes"])
                    Ld["win_scales"][0, :nw] = torch.tensor(ls["scales"])
                else:
                    assert_traj(np64(Ld["win_h"][0, :nw]), ls["H"], w.dtype, f"{tag}: window rows")
                    Ld["win_h"][0, :nw] = to_dev(ls["H"], w.dtype)
                Ld["k_cache"][0] = to_dev(ls["K"], w.dtype)
                Ld["v_cache"][0] = to_dev(ls["V"], w.dtype).permute(1, 2, 0)
                Ld["win_z"][0] = to_dev(ls["Z"], w.dtype)
                Ld["proxy_logits"][0] = torch.tensor(ls["P"], dtype=torch.float32)
            assert_traj(act_logits[0].cpu().numpy(), act_prev, w.dtype, f"step {t}: active logits")
            act_logits[0] = torch.tensor(act_prev, dtype=torch.float32)
            log(f"[trajectory] step {t} ok ({'refresh' if refresh else 'active only'})")
    finally:
        dev.close()
    log(f"[trajectory] case={case} passed")
