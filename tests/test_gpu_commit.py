"""GPU parity of Polestar-Commit: LM-head confidence of the active rows and of the
suffix rows of the final update packet, the current-block commit rule with its
drift history, and the suffix commit rule.

Inputs are seeded synthetic tensors.  Some rows are planted close to one
LM-head row so that the confidences spread over (0, 1) and straddle tau_s; one
row is planted on the mask token's row so that the argmax has to skip it.
Confidences are compared with the oracle's float64 values.  The decisions are
checked end to end: the oracle takes them from its own confidences (the rule is
a float32 comparison, taken in that precision on both sides) and the spikes and
drift history, whose inputs both sides share, must be bit-identical; a commit
mask may differ only where the oracle's confidence lies within the confidence
tolerance (2e-3 relative) of its threshold, or its spike within the matching
band around tau_d = alpha (tau_s - c)^2, and every such case is reported.  The
full-vocabulary case streams W_lm through the oracle in row chunks.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O
from tests.harness import Dev, log, np64, packet

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, batch, blk_start)
    "llada_full_vocab_batch2": (synth.shrink(synth.WORKLOADS[5], resid="raw"), 2, 512),
    "small_ragged_vocab_batch3": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64, gen=128),
                                  3, 96),
    # drift-history length h and spike weight alpha at the ends of the page's ranges
    "small_hist0_alpha2p5": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64, gen=128, hist=0,
                                          alpha=2.5), 2, 64),
    "small_hist7_alpha40": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64, gen=128, hist=7,
                                         alpha=40.0), 2, 64),
    # the other points of the page's threshold and history sweeps
    "small_hist1_taus0p7": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64, gen=128, hist=1,
                                         tau_s=0.7), 2, 64),
    "small_hist3_tausuf0p85": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64, gen=128,
                                            hist=3, tau_suf=0.85), 2, 64),
    "small_tausuf0p95": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64, gen=128,
                                      tau_suf=0.95), 2, 64),
}

CHUNK = 8192   # LM-head rows per oracle chunk
C_TOL = 2e-3   # relative tolerance of a confidence


def _check_masks(got, want, c, thr, tag, spike=None, alpha=None, spike_tol=0.0):
    """Commit masks from the two sides' confidences: equal, except where the oracle's confidence c
    is within C_TOL of its threshold (or, with spikes, the spike within the band of tau_d that the
    confidence tolerance spans, widened by ``spike_tol``, the bound on the two sides' spike
    difference when the drift itself comes from each side's own computation); such differences
    are reported."""
    got, want = np.asarray(got), np.asarray(want)
    c = np.asarray(c, dtype=np.float64)
    near = np.abs(c - thr) <= C_TOL * np.maximum(c, thr)
    if spike is not None:
        taud = alpha * (thr - c) ** 2
        band = 2 * alpha * np.abs(thr - c) * C_TOL * c + 1e-6 * np.maximum(taud, 1e-30) + spike_tol
        near |= np.abs(np.asarray(spike, np.float64) - taud) <= band
    diff = np.nonzero(got != want)[0]
    for i in diff:
        log(f"    {tag}: row {i} decided differently at a threshold (c {c[i]:.6f}, threshold {thr})")
    assert np.all(near[diff]), f"{tag}: commit masks differ away from a threshold at rows {diff[~near[diff]]}"
    return len(diff)


def _lm_logits(w, rows64: np.ndarray, eps: float) -> np.ndarray:
    """Oracle logits round(RMSNorm(x)) W_lm^T for all vocabulary ids, W_lm drawn chunk by chunk."""
    out = np.empty((rows64.shape[0], w.vocab), dtype=np.float64)
    for r0 in range(0, w.vocab, CHUNK):
        r1 = min(w.vocab, r0 + CHUNK)
        wc = np64(synth.weight_rows(w, 0, "wlm", r0, r1, device="cuda"))
        out[:, r0:r1] = O.project(rows64, wc, eps, O.storer(w.dtype))
    return out


@pytest.mark.parametrize("case", list(CASES))
def test_commit_parity(case):
    w, batch, blk_start = CASES[case]
    torch.manual_seed(0)
    dev = Dev(w, batch=batch)
    d, Bk, V = w.d, w.block, w.vocab
    mask_id = V - 1
    log(f"[commit] case={case} d={d} vocab={V} batch={batch} blk_start={blk_start}")
    try:
        g = O.window_positions(blk_start, w.n_pos, Bk, w.win_prefix, w.win_suffix)
        n_pre = int(np.sum(g < blk_start))
        n_win = len(g)
        n_suf = n_win - n_pre
        seed = w.seed(0)
        # LM head on the GPU
        wlm = synth.weight(w, 0, "wlm", device="cuda")
        w_lm = dev.pack(B.W_LM, wlm)
        # active rows: random, with planted rows near W_lm rows (confidences spread over (0, 1))
        # x = sqrt(d) W_lm[v] + l g (g ~ N(0, 1) per element) gives the planted logit about
        # sqrt(d) / sqrt(1 + l^2) against N(0, 1) logits elsewhere; noise_for(tau) puts c near tau.
        h_fin = synth.tensor(w, (90, 1), (batch, Bk, d), 1.0, device="cuda", dtype="f32")

        def noise_for(tau):
            target = np.log(V) + 0.5 + np.log(tau / (1.0 - tau))
            return np.sqrt(max((np.sqrt(d) / target) ** 2 - 1.0, 0.01))

        l0, l_suf = noise_for(w.tau_s), noise_for(w.tau_suf)
        for b in range(batch):
            for i, f in enumerate([0.6, 0.85, 0.94, 0.99, 1.04, 1.11, 1.33, 1.7]):
                j = (3 * i + b) % (Bk - 1)
                v = int(synth.hash32_int(seed + 31 * b + i) % (V - 1))
                h_fin[b, j] = wlm[v].float() * np.sqrt(d) + (l0 * f) * h_fin[b, j]
            h_fin[b, Bk - 1] = wlm[mask_id].float() * np.sqrt(d)   # argmax must skip the mask id
        h_fin = h_fin.to(torch.bfloat16)
        # final update packet: ascending window rows, a mix of prefix and suffix rows
        win_max = dev.win_max
        u_rows = synth.tensor(w, (90, 2), (batch, win_max, d), 1.0, device="cuda", dtype="f32")
        u_idx = torch.full((batch, win_max), -1, dtype=torch.int32)
        u_cnt = torch.zeros(batch, dtype=torch.int32)
        rng = np.random.default_rng(seed)
        for b in range(batch):
            pick = np.sort(rng.choice(n_win, size=min(n_win, 12 + 7 * b), replace=False))
            u_idx[b, :len(pick)] = torch.tensor(pick, dtype=torch.int32)
            u_cnt[b] = len(pick)
            for t, wr in enumerate(pick[::3]):      # suffix/prefix packet rows with c spread around tau_suf
                v = int(synth.hash32_int(seed + 7 * b + t + 1000) % (V - 1))
                r = int(np.nonzero(pick == wr)[0][0])
                f = (0.05, 0.8, 0.95, 1.05, 1.25)[t % 5]
                u_rows[b, r] = wlm[v].float() * np.sqrt(d) + (l_suf * f) * u_rows[b, r]
        u_rows = u_rows.to(torch.bfloat16)
        u_idx_d, u_cnt_d = u_idx.cuda(), u_cnt.cuda()
        # drift, masks, history
        delta = (synth.tensor(w, (90, 3), (batch, Bk), 1.0, device="cuda").abs() * 2.0).contiguous()
        act_mask = torch.tensor(rng.integers(0, 2, size=(batch, Bk)), dtype=torch.uint8)
        act_mask[:, :8] = 1
        suf_mask = torch.tensor(rng.integers(0, 2, size=(batch, max(w.win_suffix, 1))), dtype=torch.uint8)
        H = max(w.hist, 1)
        hist_vals = synth.tensor(w, (90, 4), (batch, Bk, H), 1.0, device="cuda").abs().contiguous()
        hist_cnt = torch.tensor(rng.integers(0, w.hist + 1, size=(batch, Bk)), dtype=torch.int32)
        hv0, hc0 = hist_vals.cpu().numpy().copy(), hist_cnt.numpy().copy()
        outs = dict(commit_active=torch.zeros(batch, Bk, dtype=torch.uint8),
                    commit_suffix=torch.zeros(batch, w.win_suffix, dtype=torch.uint8),
                    conf_active=torch.zeros(batch, Bk), yhat=torch.zeros(batch, Bk, dtype=torch.int32),
                    spike=torch.zeros(batch, Bk), conf_suffix=torch.zeros(batch, w.win_suffix))
        outs = {k: v.cuda() for k, v in outs.items()}
        hist_cnt_d = hist_cnt.cuda()
        act_mask_d, suf_mask_d = act_mask.cuda(), suf_mask.cuda()
        B.polestar_commit(dev.h, blk_start, w_lm, h_fin, packet(u_rows, u_idx_d, u_cnt_d), delta, act_mask_d,
                          suf_mask_d, hist_vals, hist_cnt_d, outs["commit_active"], outs["commit_suffix"],
                          outs["conf_active"], outs["yhat"], outs["spike"], outs["conf_suffix"], dev.ws,
                          dev.ws_bytes)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in outs.items()}
        for b in range(batch):
            # oracle confidences of the active rows and the suffix packet rows
            cnt = int(u_cnt[b])
            idx = u_idx[b, :cnt].numpy()
            suf_r = [r for r in range(cnt) if idx[r] >= n_pre]
            rows = np.concatenate([np64(h_fin[b]), np64(u_rows[b])[suf_r]], axis=0)
            lg = _lm_logits(w, rows, w.rms_eps)
            c, yhat = O.confidence_from_logits(lg, mask_id)
            ca, ya = c[:Bk], yhat[:Bk]
            err = np.abs(got["conf_active"][b] - ca) / np.maximum(ca, 1e-30)
            log(f"    seq {b}: active confidences {np.round(ca[:8], 3)} max rel err {err.max():.2e}")
            assert err.max() <= 2e-3, f"seq {b}: confidence rel err {err.max():.3e}"
            assert np.array_equal(got["yhat"][b], ya), f"seq {b}: argmax ids differ"
            assert got["yhat"][b][Bk - 1] != mask_id
            assert (ca >= w.tau_s).any() and (ca < w.tau_s).any(), "planted rows should straddle tau_s"
            # the rule on the oracle's own confidences: masks end to end; spikes and history, whose
            # inputs both sides share, bit-identical
            com, sp, _, hv, hc = O.commit_decide(np64(delta[b]), ca.astype(np.float32), act_mask[b].numpy(),
                                                 hv0[b], hc0[b], w.hist, w.alpha, w.tau_s)
            _check_masks(got["commit_active"][b], com, ca, w.tau_s, f"seq {b} active", sp, w.alpha)
            assert np.array_equal(got["spike"][b].astype(np.float32), sp), f"seq {b}: spike differs"
            assert np.array_equal(hist_cnt_d[b].cpu().numpy(), hc)
            assert np.array_equal(hist_vals[b].cpu().numpy().reshape(Bk, -1)[:, :w.hist],
                                  hv.reshape(Bk, -1)[:, :w.hist].astype(np.float32))
            # suffix rows
            cs = c[Bk:]
            conf_suf = np.zeros(w.win_suffix, dtype=np.float64)
            elig = np.zeros(w.win_suffix, dtype=bool)
            for t, r in enumerate(suf_r):
                slot = int(idx[r]) - n_pre
                err = abs(got["conf_suffix"][b][slot] - cs[t]) / max(cs[t], 1e-30)
                assert err <= C_TOL, f"seq {b}: suffix confidence rel err {err:.3e}"
                conf_suf[slot] = cs[t]
                elig[slot] = suf_mask[b, slot] != 0
            want = O.suffix_commit(conf_suf.astype(np.float32), elig, w.tau_suf)
            _check_masks(got["commit_suffix"][b], want, conf_suf, w.tau_suf, f"seq {b} suffix")
            log(f"    seq {b}: {int(com.sum())} active commits, {int(want.sum())} suffix commits, "
                f"{len(suf_r)} suffix packet rows of {n_suf}")
    finally:
        dev.close()
    log(f"[commit] case={case} passed")


ENTRY_CASES = {
    # name: (workload, batch, blk_start)
    "llada_full_vocab_entry_batch2": (synth.shrink(synth.WORKLOADS[5], resid="raw"), 2, 512),
    "small_ragged_vocab_entry_suffix_cut": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64,
                                                         gen=128), 2, 144),
    "small_ragged_vocab_entry_at_end": (synth.shrink(synth.WORKLOADS[1], dtype="bf16", vocab=1008, prompt=64,
                                                     gen=128), 1, 160),
}


@pytest.mark.parametrize("case", list(ENTRY_CASES))
def test_entry_commit_parity(case):
    """Block-entry commit: confidences of the active rows and of every suffix window row, read at
    their positions in the rows of all positions; decisions by confidence alone."""
    w, batch, blk_start = ENTRY_CASES[case]
    dev = Dev(w, batch=batch)
    d, Bk, V, n = w.d, w.block, w.vocab, w.n_pos
    mask_id = V - 1
    log(f"[entry-commit] case={case} d={d} vocab={V} batch={batch} blk_start={blk_start}")
    try:
        g = O.window_positions(blk_start, n, Bk, w.win_prefix, w.win_suffix)
        n_suf = int(np.sum(g >= blk_start + Bk))
        seed = w.seed(0)
        wlm = synth.weight(w, 0, "wlm", device="cuda")
        w_lm = dev.pack(B.W_LM, wlm)
        # rows of every position, with planted rows near W_lm rows in the active block and suffix
        h_full = synth.tensor(w, (91, 1), (batch, n, d), 1.0, device="cuda", dtype="f32")
        target = np.log(V) + 0.5 + np.log(9.0)
        l0 = np.sqrt(max((np.sqrt(d) / target) ** 2 - 1.0, 0.01))
        rows_of = np.arange(blk_start, blk_start + Bk + n_suf)
        for b in range(batch):
            for i, f in enumerate([0.6, 0.85, 0.94, 0.99, 1.04, 1.11, 1.33, 1.7, 0.9, 1.0]):
                p = int(rows_of[(5 * i + 2 * b) % len(rows_of)])
                v = int(synth.hash32_int(seed + 41 * b + i) % (V - 1))
                h_full[b, p] = wlm[v].float() * np.sqrt(d) + (l0 * f) * h_full[b, p]
            h_full[b, blk_start] = wlm[mask_id].float() * np.sqrt(d)   # argmax must skip the mask id
        h_full = h_full.to(torch.bfloat16).contiguous()
        rng = np.random.default_rng(seed + 5)
        act_mask = torch.tensor(rng.integers(0, 2, size=(batch, Bk)), dtype=torch.uint8)
        act_mask[:, :4] = 1
        suf_mask = torch.tensor(rng.integers(0, 2, size=(batch, max(w.win_suffix, 1))), dtype=torch.uint8)
        outs = dict(commit_active=torch.zeros(batch, Bk, dtype=torch.uint8),
                    commit_suffix=torch.full((batch, w.win_suffix), 7, dtype=torch.uint8),
                    conf_active=torch.zeros(batch, Bk), yhat=torch.zeros(batch, Bk, dtype=torch.int32),
                    conf_suffix=torch.full((batch, w.win_suffix), -1.0))
        outs = {k: v.cuda() for k, v in outs.items()}
        B.polestar_entry_commit(dev.h, blk_start, w_lm, h_full, act_mask.cuda(), suf_mask.cuda(),
                                outs["commit_active"], outs["commit_suffix"], outs["conf_active"], outs["yhat"],
                                outs["conf_suffix"], dev.ws, dev.ws_bytes)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in outs.items()}
        for b in range(batch):
            lg = _lm_logits(w, np64(h_full[b, rows_of]), w.rms_eps)
            c, yhat = O.confidence_from_logits(lg, mask_id)
            ca, cs = c[:Bk], c[Bk:]
            err = np.abs(got["conf_active"][b] - ca) / np.maximum(ca, 1e-30)
            assert err.max() <= 2e-3, f"seq {b}: active confidence rel err {err.max():.3e}"
            assert np.array_equal(got["yhat"][b], yhat[:Bk]), f"seq {b}: argmax ids differ"
            assert got["yhat"][b][0] != mask_id
            assert (ca >= w.tau_s).any() or (cs >= w.tau_suf).any(), "planted rows should reach the thresholds"
            es = np.abs(got["conf_suffix"][b][:n_suf] - cs) / np.maximum(cs, 1e-30)
            assert es.size == 0 or es.max() <= 2e-3, f"seq {b}: suffix confidence rel err {es.max():.3e}"
            assert np.all(got["conf_suffix"][b][n_suf:] == 0) and np.all(got["commit_suffix"][b][n_suf:] == 0)
            # the rule on the oracle's own confidences, masks end to end
            _check_masks(got["commit_active"][b], O.entry_commit(ca.astype(np.float32), act_mask[b].numpy(), w.tau_s),
                         ca, w.tau_s, f"seq {b} entry active")
            _check_masks(got["commit_suffix"][b][:n_suf],
                         O.entry_commit(cs.astype(np.float32), suf_mask[b, :n_suf].numpy(), w.tau_suf), cs, w.tau_suf,
                         f"seq {b} entry suffix")
            log(f"    seq {b}: {int(got['commit_active'][b].sum())} active and "
                f"{int(got['commit_suffix'][b].sum())} suffix commits of {Bk} + {n_suf} rows")
    finally:
        dev.close()
    log(f"[entry-commit] case={case} passed")
