"""Degenerate cases of the drift step on the GPU, from planted state [Polestar §4.1, Eq. 4 and
the top-k cluster selection]:

1. exact drift ties: window rows in pairs of clusters with identical members (in the same order)
   and identical previous proxy logits, so that both sides compute bit-equal drifts for the two
   clusters of a pair; with k = 3 one pair straddles the selection boundary and the lower
   cluster index must win;
2. an empty cluster: its centroid is kept by the update, its drift is still formed (its previous
   logits are planted far from the current ones so that it is selected), and it adds no rows to S.

The window update runs without an incoming packet (every centroid is recomputed from its members).
D is compared with the oracle under the per-call rule (2e-3 plus the oracle-derived allowance),
top-k and S exactly.  Fewer window rows than clusters (n_Omega < K) runs through the layer
parity cases, where the block-entry clustering itself sees it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O
from tests import flips as FL
from tests.harness import (Dev, assert_close, assert_stored, check_topk, layer_struct, log, np64, oracle_weights,
                           packed_layer, packet, to_dev, weights)

pytestmark = pytest.mark.gpu

W_EDGE = synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=128, gen=128, top_k=3)


def _planted_state(w, scenario):
    """Oracle layer state with planted window rows, labels and previous proxy logits."""
    cfg = O.Cfg.from_workload(w, top_k=w.top_k)
    st = cfg.st
    n, d, hq, hkv, dh, K = w.n_pos, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.n_clusters
    blk = w.prompt
    wpos = O.window_positions(blk, n, w.block, w.win_prefix, w.win_suffix)
    nw = len(wpos)
    g = nw // K                                     # rows per cluster
    t = lambda tag, shape, std=1.0, dtype=w.dtype: np64(synth.tensor(w, (70,) + tag, shape, std, 0, "cpu", dtype))
    M = np.minimum(np.arange(nw) // g, K - 1).astype(np.int32)
    P = O.round_f32(t((1,), (K, hq, n), 3.0, "f32"))
    if scenario == "ties":
        base = t((2,), (K // 2, g, d))
        H = np.zeros((nw, d))
        for c in range(K):
            rows = np.nonzero(M == c)[0]
            H[rows] = base[c // 2][: len(rows)]
        for c in range(1, K, 2):
            P[c] = P[c - 1]                         # twin clusters share their previous logits
    else:   # an empty cluster 5: its rows join cluster 4; its previous logits far from any current ones
        H = t((3,), (nw, d))
        M[M == 5] = 4
        P[5] = O.round_f32(t((4,), (hq, n), 12.0, "f32"))
    Z = st(O.unit_rows(t((5,), (K, d))))
    ls = {"K": t((6,), (n, hkv, dh)), "V": t((7,), (n, hkv, dh)), "Z": Z, "M": M, "H": H, "P": P}
    return cfg, ls, wpos


@pytest.mark.parametrize("scenario", ["ties", "empty_cluster"])
def test_planted_drift_degenerate_cases(scenario):
    w = W_EDGE
    log(f"[edge] scenario={scenario} d={w.d} n={w.n_pos} K={w.n_clusters} k={w.top_k}")
    dev = Dev(w, batch=1, vocab=0)
    try:
        cfg, ls, wpos = _planted_state(w, scenario)
        st = cfg.st
        n, d, hq, dh, K, Bk = w.n_pos, w.d, w.n_heads, w.head_dim, w.n_clusters, w.block
        blk = w.prompt
        nw, WM = len(wpos), dev.win_max
        Wd = weights(w, 0)
        Wo = oracle_weights(Wd)
        Ld = packed_layer(dev, Wd)
        del Wd
        Ld["k_cache"] = to_dev(ls["K"], w.dtype)[None].contiguous()
        Ld["v_cache"] = to_dev(ls["V"], w.dtype).permute(1, 2, 0)[None].contiguous()
        Ld["win_z"] = to_dev(ls["Z"], w.dtype)[None].contiguous()
        m = torch.zeros(1, WM, dtype=torch.int32, device="cuda")
        m[0, :nw] = torch.tensor(ls["M"])
        Ld["win_m"] = m
        Ld["proxy_logits"] = torch.tensor(ls["P"], dtype=torch.float32, device="cuda")[None].contiguous()
        hw = dev.zeros(1, WM, d)
        hw[0, :nw] = to_dev(ls["H"], w.dtype)
        Ld["win_h"] = hw
        Ls = layer_struct(Ld)
        z_before = Ld["win_z"].clone()

        # window update without a packet, then the drift call
        B.polestar_cluster(dev.h, B.CLUSTER_UPDATE, Ls, blk, None, None, None, None, dev.ws, dev.ws_bytes)
        h_act = to_dev(np64(synth.tensor(w, (70, 8), (Bk, d), 1.0, 0, "cpu", w.dtype)), w.dtype)[None].contiguous()
        D = torch.zeros(1, K, dtype=torch.float32, device="cuda")
        topk = torch.zeros(1, w.top_k, dtype=torch.int32, device="cuda")
        sel_idx = torch.zeros(1, WM, dtype=torch.int32, device="cuda")
        sel_cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.polestar_drift(dev.h, B.DRIFT_REFRESH, Ls, blk, h_act, None, D, topk, packet(None, sel_idx, sel_cnt), None,
                         None, dev.ws, dev.ws_bytes)
        torch.cuda.synchronize()

        cu = O.cluster_update(ls, cfg)
        assert_stored(np64(Ld["win_z"][0]), ls["Z"], w.dtype, "updated centroids")
        P_before = np.array(ls["P"], copy=True)
        ha = np64(h_act[0])
        dr = O.drift_layer(ls, Wo, cfg, blk, ha, cu["h"], cu["patched"], True)
        al = FL.drift_call_allow(O, cfg, Wo, blk, ha, cu["h"], cu["patched"], ls["Z"], ls["K"], ls["V"],
                                 dr["proxy_q"], dr["proxy_keys"], P_before)
        Dg = D[0].cpu().numpy()
        tg = topk[0].cpu().numpy()
        log(f"    D gpu {np.round(Dg, 5).tolist()}\n    D oracle {np.round(dr['D'], 5).tolist()}\n"
            f"    top-k gpu {tg.tolist()} oracle {dr['topk'].tolist()}")
        assert_close(Dg, dr["D"], "cluster drift D", allow=al["D"])
        if scenario == "ties":
            for c in range(0, K, 2):
                assert Dg[c] == Dg[c + 1], f"GPU drifts of twin clusters {c}, {c + 1} differ"
                assert dr["D"][c] == dr["D"][c + 1], f"oracle drifts of twin clusters {c}, {c + 1} differ"
            # the pair that straddles the boundary gives its lower index
            chosen = set(tg.tolist())
            split = [c for c in range(0, K, 2) if (c in chosen) != (c + 1 in chosen)]
            assert len(split) == 1 and split[0] in chosen, f"tie at the boundary not broken to the lower index: {tg}"
            log(f"    pair ({split[0]}, {split[0] + 1}) straddles the top-{w.top_k} boundary: {split[0]} chosen")
        else:
            z1 = Ld["win_z"][0].cpu()
            assert torch.equal(z1[5], z_before[0, 5].cpu()), "empty cluster's centroid changed"
            assert 5 in tg.tolist() and 5 in dr["topk"].tolist(), "the planted empty cluster should be selected"
        assert check_topk(tg, Dg, dr["D"], dr["topk"], w.top_k, min(K, nw), f"edge {scenario}", al["D"]), \
            "top-k near-tie"
        cnt = int(sel_cnt[0])
        S = sel_idx[0, :cnt].cpu().numpy()
        assert np.array_equal(S, dr["S"]), "selected rows S differ"
        assert np.array_equal(S, np.nonzero(np.isin(ls["M"], tg))[0]), "S is not the members of the chosen clusters"
        log(f"    |S| = {cnt}")
    finally:
        dev.close()
    log(f"[edge] scenario={scenario} passed")
