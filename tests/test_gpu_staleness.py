"""KV-cache staleness on the GPU [App. C.2 of the Polestar page] and the
selection-accuracy measurement of §3 / Fig. 6(a).

1. The staleness kernel against the oracle's E_i on random caches with fresh,
   opposite and zero rows.
2. A free-running bf16 trajectory (oracle block entry, then GPU steps): at every
   refresh step and layer, right after the drift call picked S, the caches are
   compared with a full recompute of the current sequence (the oracle's dense
   forward): E_i of every position from the GPU kernel (checked against the
   oracle), and the share of the true top-quarter most stale window positions
   that S contains, beside a random choice of the same size.  With synthetic
   weights the numbers say nothing about trained models; the test checks the
   measurement and reports it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O
from tests.harness import Dev, layer_struct, log, np64, packed_layer, packet, to_dev, weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_staleness_kernel_matches_oracle(dtype):
    w = synth.shrink(synth.WORKLOADS[1], dtype=dtype, n_kv_heads=2, n_heads=4)
    log(f"[staleness] kernel dtype={dtype} n={w.n_pos} hkv={w.n_kv_heads}")
    dev = Dev(w, batch=2, vocab=0)
    try:
        n, H, dh = w.n_pos, w.n_kv_heads, w.head_dim
        rng = np.random.default_rng(71)
        k, v = rng.normal(size=(2, n, H, dh)), rng.normal(size=(2, n, H, dh))
        kr, vr = rng.normal(size=(2, n, H, dh)), rng.normal(size=(2, n, H, dh))
        kr[:, :5], vr[:, :5] = k[:, :5], v[:, :5]          # fresh rows
        kr[:, 5:9], vr[:, 5:9] = -k[:, 5:9], -v[:, 5:9]    # opposite rows
        k[:, 9:11] = 0.0                                   # zero K rows
        kd = [to_dev(x, dtype) for x in (k, kr)]
        vd = [to_dev(x, dtype).permute(0, 2, 3, 1).contiguous() for x in (v, vr)]   # [b, H, dh, n]
        E = torch.zeros(2, n, dtype=torch.float32, device="cuda")
        B.polestar_kv_staleness(dev.h, kd[0], vd[0], kd[1], vd[1], E)
        torch.cuda.synchronize()
        for b in range(2):
            # the oracle on the stored (rounded) values
            ref = O.kv_staleness(np64(kd[0][b]), np64(vd[0][b].permute(2, 0, 1)), np64(kd[1][b]),
                                 np64(vd[1][b].permute(2, 0, 1)))
            got = E[b].cpu().numpy()
            assert np.max(np.abs(got - ref)) < 1e-5, f"E_i differs by {np.max(np.abs(got - ref)):.2e}"
            assert np.allclose(got[:5], 0.0, atol=1e-6) and np.allclose(got[5:9], 2.0, atol=1e-6)
    finally:
        dev.close()


ATTEND_CASES = {
    # name: (workload, batch, rows, q row stride padding)
    "tiny_f32_gqa": (synth.shrink(synth.WORKLOADS[1], n_heads=4, n_kv_heads=2), 2, 40, 0),
    "tiny_bf16_padded_rows": (synth.shrink(synth.WORKLOADS[1], dtype="bf16"), 1, 96, 64),
    "llada_bf16_n1024": (synth.shrink(synth.WORKLOADS[3], n_layers=1), 1, 96, 0),
    "dream_gqa_bf16": (synth.shrink(synth.WORKLOADS[4], n_layers=1), 1, 64, 0),
    "tiny_bf16_n2048": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", prompt=1024, gen=1024), 1, 48, 0),
}


@pytest.mark.parametrize("case", list(ATTEND_CASES))
def test_attended_change_kernel_matches_oracle(case):
    """Most-attended token and its cosine change: the token exact where the oracle's head-mean
    probabilities separate the top two positions by more than 1e-5 of the largest (else the
    GPU's token must be one of the near-maximal ones), the score within 2e-3 of the oracle's
    score of the GPU's token (floor 1e-4)."""
    w, batch, rows, pad = ATTEND_CASES[case]
    n, hq, hkv, dh = w.n_pos, w.n_heads, w.n_kv_heads, w.head_dim
    log(f"[attended] case={case} n={n} heads={hq}/{hkv} dh={dh} rows={rows} batch={batch} dtype={w.dtype}")
    dev = Dev(w, batch=batch, vocab=0)
    try:
        q_ld = hq * dh + pad
        q = synth.tensor(w, (80, 1), (batch, rows, q_ld), 1.0, 0, "cuda", "f32")
        k = synth.tensor(w, (80, 2), (batch, n, hkv, dh), 1.0, 0, "cuda", w.dtype)
        # reference keys: unchanged, scaled, perturbed and fresh rows
        kr = k.clone()
        pert = synth.tensor(w, (80, 3), (batch, n, hkv, dh), 1.0, 0, "cuda", "f32")
        sel = torch.arange(n, device="cuda") % 4
        kr[:, sel == 1] = (k[:, sel == 1].float() * 2.0).to(k.dtype)
        kr[:, sel == 2] = (k[:, sel == 2].float() + 0.3 * pert[:, sel == 2]).to(k.dtype)
        kr[:, sel == 3] = pert[:, sel == 3].to(k.dtype)
        # a few queries aimed at chosen keys, so that some rows have a dominant token
        for b in range(batch):
            for r in range(0, rows, 5):
                j = int(synth.hash32_int(w.seed(0) + 13 * b + r) % n)
                for h in range(hq):
                    q[b, r, h * dh:(h + 1) * dh] = 3.0 * k[b, j, (h * hkv) // hq].float()
        top = torch.zeros(batch, rows, dtype=torch.int32, device="cuda")
        score = torch.zeros(batch, rows, dtype=torch.float32, device="cuda")
        B.polestar_attended_change(dev.h, q, rows, q_ld, rows * q_ld, k, kr, top, score)
        torch.cuda.synchronize()
        near = 0
        for b in range(batch):
            qo = np64(q[b, :, : hq * dh]).reshape(rows, hq, dh)
            ko, kro = np64(k[b]), np64(kr[b])
            j_or, s_or, A = O.attended_token_change(qo, ko, kro, hq, hkv)
            jg = top[b].cpu().numpy()
            sg = score[b].cpu().numpy()
            amax = A.max(axis=1)
            srt = np.sort(A, axis=1)
            gap = srt[:, -1] - srt[:, -2]
            sep = gap > 1e-5 * amax
            assert np.array_equal(jg[sep], j_or[sep]), f"seq {b}: most-attended tokens differ"
            ok = A[np.arange(rows), jg] >= amax - 1e-5 * amax
            assert ok.all(), f"seq {b}: GPU token not among the near-maximal positions"
            near += int((~sep).sum())
            s_at = 1.0 - np.mean(O.cosine(ko[jg], kro[jg]), axis=-1)   # oracle score of the GPU's token
            err = np.abs(sg - s_at) / np.maximum(np.abs(s_at), 1e-4)
            assert err.max() <= 2e-3, f"seq {b}: score rel err {err.max():.2e}"
            log(f"    seq {b}: {int(sep.sum())} rows with a separated maximum, scores in "
                f"[{sg.min():.3f}, {sg.max():.3f}], max rel err {err.max():.2e}")
        log(f"[attended] case={case} passed ({near} near-tied rows checked as valid choices)")
    finally:
        dev.close()


def test_staleness_and_selection_accuracy_of_the_drift_policy():
    w = synth.shrink(synth.WORKLOADS[1], dtype="bf16", top_k=2)     # k/K = 1/4: the page's top quarter
    n_layers, steps = 2, 6
    log(f"[staleness] trajectory d={w.d} n={w.n_pos} layers={n_layers} steps={steps} K={w.n_clusters} k={w.top_k}")
    dev = Dev(w, batch=1, vocab=0)
    cfg = O.Cfg.from_workload(w, top_k=w.top_k)
    st = cfg.st
    n, d, Bk, K = w.n_pos, w.d, w.block, w.n_clusters
    blk_start = w.prompt
    wpos = np.asarray(O.window_positions(blk_start, n, Bk, w.win_prefix, w.win_suffix))
    nw, WM = len(wpos), dev.win_max
    rng = np.random.default_rng(5)
    acc_kl, acc_rand = [], []
    try:
        Wd = [weights(w, l) for l in range(n_layers)]
        Wo = [{k_: np64(v_) for k_, v_ in W.items()} for W in Wd]
        P = [packed_layer(dev, W) for W in Wd]
        del Wd
        h0 = st(np64(synth.embeddings(w)))
        Hs, Ks, Vs, _ = O.full_forward(h0, Wo, cfg)
        L, Ls = [], []
        for l in range(n_layers):
            ls = O.block_entry_layer_state(Hs[l], Ks[l], Vs[l], Wo[l]["wq"], cfg, blk_start,
                                           synth.kmeans_init(w, nw, l, 0))
            Ld = dict(P[l])
            Ld["k_cache"] = to_dev(ls["K"], w.dtype)[None].contiguous()
            Ld["v_cache"] = to_dev(ls["V"], w.dtype).permute(1, 2, 0)[None].contiguous()
            Ld["win_z"] = to_dev(ls["Z"], w.dtype)[None].contiguous()
            m = torch.zeros(1, WM, dtype=torch.int32, device="cuda")
            m[0, :nw] = torch.tensor(ls["M"], dtype=torch.int32)
            Ld["win_m"] = m
            Ld["proxy_logits"] = torch.tensor(ls["P"], dtype=torch.float32, device="cuda")[None].contiguous()
            hw = dev.zeros(1, WM, d)
            hw[0, :nw] = to_dev(ls["H"], w.dtype)
            Ld["win_h"] = hw
            L.append(Ld)
            Ls.append(layer_struct(Ld))
        h_act = [dev.zeros(1, Bk, d) for _ in range(2)]
        pk_rows = [dev.zeros(1, WM, d) for _ in range(2)]
        pk_idx = [torch.zeros(1, WM, dtype=torch.int32, device="cuda") for _ in range(2)]
        pk_cnt = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]
        pks = [packet(pk_rows[i], pk_idx[i], pk_cnt[i]) for i in range(2)]
        D = torch.zeros(1, K, dtype=torch.float32, device="cuda")
        topk = torch.zeros(1, w.top_k, dtype=torch.int32, device="cuda")
        E = torch.zeros(1, n, dtype=torch.float32, device="cuda")
        for t in range(steps):
            noise = np64(synth.tensor(w, (77, t), (Bk, d), np.sqrt(w.noise_var)))
            x = st(h0[blk_start: blk_start + Bk] + noise)
            h_act[0][0] = to_dev(x, w.dtype)
            # the full recompute of the current sequence: the entry inputs with this step's block
            hcur = h0.copy()
            hcur[blk_start: blk_start + Bk] = x
            _, Kr, Vr, _ = O.full_forward(hcur, Wo, cfg)
            cur, pk, u_in = 0, 0, None
            for l in range(n_layers):
                B.polestar_cluster(dev.h, B.CLUSTER_UPDATE, Ls[l], blk_start, u_in, None, None, None, dev.ws,
                                   dev.ws_bytes)
                sel = pks[pk]
                B.polestar_drift(dev.h, B.DRIFT_REFRESH, Ls[l], blk_start, h_act[cur], u_in, D, topk, sel, None,
                                 None, dev.ws, dev.ws_bytes)
                # staleness of this layer's cache at the moment S is chosen
                kr = to_dev(Kr[l], w.dtype)[None].contiguous()
                vr = to_dev(Vr[l], w.dtype).permute(1, 2, 0)[None].contiguous()
                B.polestar_kv_staleness(dev.h, L[l]["k_cache"], L[l]["v_cache"], kr, vr, E)
                torch.cuda.synchronize()
                e = E[0].cpu().numpy()
                ref = O.kv_staleness(np64(L[l]["k_cache"][0]), np64(L[l]["v_cache"][0].permute(2, 0, 1)),
                                     np64(kr[0]), np64(vr[0].permute(2, 0, 1)))
                assert np.max(np.abs(e - ref)) < 1e-5
                assert np.all(np.isfinite(e)) and e.min() > -1e-5 and e.max() < 2 + 1e-5
                cnt = int(pk_cnt[pk][0])
                S = pk_idx[pk][0, :cnt].cpu().numpy()
                ew = e[wpos]
                if cnt:
                    acc_kl.append(O.selection_accuracy(S, ew))
                    acc_rand.append(O.selection_accuracy(rng.choice(nw, size=cnt, replace=False), ew))
                log(f"    step {t} layer {l}: |S| = {cnt}, window E mean {ew.mean():.4f} max {ew.max():.4f}, "
                    f"drift-policy accuracy {acc_kl[-1] if cnt else float('nan'):.2f}")
                B.polestar_refresh(dev.h, Ls[l], blk_start, h_act[cur], sel, None, None, None, h_act[1 - cur],
                                   pk_rows[pk], dev.ws, dev.ws_bytes)
                u_in = sel
                cur, pk = 1 - cur, 1 - pk
        torch.cuda.synchronize()
        assert acc_kl, "no refresh selected any row"
        log(f"[staleness] top-quarter selection accuracy over {len(acc_kl)} (step, layer) points: "
            f"KL drift {np.mean(acc_kl):.3f}, random {np.mean(acc_rand):.3f}")
    finally:
        dev.close()
