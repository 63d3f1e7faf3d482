"""Admissible rounding alternatives and their first-order effect, from the oracle alone.

A value that the method stores in bfloat16 (a K/V cache row, a projection input
round(RMSNorm(x)), a layer output) and whose exact value lies within a hair of a
bf16 rounding midpoint may be rounded either way by a correct float32
implementation: its float32 value and the oracle's float64 value differ by about
1e-6 relative, which is enough to decide such a tie differently.  Both roundings
are correct results of the method.  When such a stored value feeds a later
computation in the same call (the attention reads the K/V rows the call has just
stored), the later values may differ from the oracle's by the effect of the
other rounding.

This module computes, from the oracle's pre-rounding values only (never from
GPU output), an upper bound of that effect to first order:
  * ``stored_dev``: per stored element, the admissible deviation of the stored
    value (one ulp where the pre-rounding value is within ``TIE`` ulp of a
    midpoint, plus any admissible deviation already carried by the pre-rounding
    value itself);
  * ``proj_dev``: a projection's output deviation, |W| applied to its inputs';
  * ``attn_dev``: logits, attention outputs and KL drift of query rows over a
    cache whose rows carry stored deviations.
The parity tests add these bounds (times ``SAFETY``, for the neglected second
order) to the 2e-3 rule and report how many elements needed them.
"""
from __future__ import annotations

import math

import numpy as np

TIE = 1e-3      # a pre-rounding value this close to a midpoint (in ulps) may round either way
SAFETY = 2.0    # margin over the first-order bound
EPS32 = 2.0 ** -22   # relative float32 error of a GPU value before storage, generously


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage dtype's values at |x| (bf16: 8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(x > 0, x, 1.0))          # x = m 2^e, m in [0.5, 1)
    bits = 8 if dtype == "bf16" else 24
    return np.where(x > 0, np.ldexp(1.0, e - bits), 0.0)


def stored_dev(pre: np.ndarray, dtype: str, pre_dev=None) -> np.ndarray:
    """Admissible |GPU stored - oracle stored| per element of a stored tensor whose oracle value
    before rounding is ``pre`` and whose GPU value before rounding may differ from it by
    ``pre_dev`` (admissible deviations upstream) plus float32 error."""
    pre = np.asarray(pre, dtype=np.float64)
    d0 = np.zeros_like(pre) if pre_dev is None else np.asarray(pre_dev, dtype=np.float64)
    if dtype != "bf16":
        return d0
    u = ulp(pre, dtype)
    frac = np.abs(pre) / np.where(u > 0, u, 1.0)
    to_mid = np.abs(frac - np.floor(frac) - 0.5) * u        # distance to the nearest midpoint
    reach = d0 + (TIE * u) + EPS32 * np.abs(pre)
    return d0 + np.where(to_mid <= reach, u, 0.0)


def rms_dev(x: np.ndarray, dx: np.ndarray, eps: float) -> np.ndarray:
    """Deviation of RMSNorm(x) (unit gain) for input deviations dx, to first order:
    |d(x/r)| <= |dx|/r + |x| sum|x dx| / (d r^3)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return np.abs(dx) / r + np.abs(x) * np.sum(np.abs(x * dx), axis=-1, keepdims=True) / (x.shape[-1] * r ** 3)


def proj_dev(dx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """|W| |dx|: deviation of x W^T for input deviations dx (rows on the last axis)."""
    return np.abs(np.asarray(dx, dtype=np.float64)) @ np.abs(np.asarray(w, dtype=np.float64)).T


def norm_in_dev(x: np.ndarray, eps: float, dtype: str, dx=None) -> np.ndarray:
    """Deviation of the projection input round(RMSNorm(x)) (the rounding point of every
    projection of a stored row) for input deviations dx (None: the inputs are shared)."""
    x = np.asarray(x, dtype=np.float64)
    a = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    da = None if dx is None else rms_dev(x, dx, eps)
    return stored_dev(a, dtype, da)


def attn_dev(q, K, V, dq, dK, dV, hq, hkv, P_prev=None, keys=None):
    """First-order deviation bounds of softmax attention of query rows q [R, Hq, dh] over the
    cache K, V [n, Hkv, dh] (oracle values) when q, K, V may deviate by dq, dK, dV (>= 0, same
    shapes; zero where both sides share the value).  keys: the key positions attended (None: all).
    Returns (dlogits [R, Hq, nk], dout [R, Hq, dh], dkl [R, Hq] against P_prev [R, Hq, nk] when
    given, else None)."""
    q, dq = np.asarray(q, np.float64), np.asarray(dq, np.float64)
    if keys is not None:
        K, V, dK, dV = K[keys], V[keys], dK[keys], dV[keys]
    g = (np.arange(hq) * hkv) // hq
    Kh = np.asarray(K, np.float64)[:, g, :].transpose(1, 0, 2)       # [Hq, n, dh]
    Vh = np.asarray(V, np.float64)[:, g, :].transpose(1, 0, 2)
    dKh = np.asarray(dK, np.float64)[:, g, :].transpose(1, 0, 2)
    dVh = np.asarray(dV, np.float64)[:, g, :].transpose(1, 0, 2)
    qh, dqh = q.transpose(1, 0, 2), dq.transpose(1, 0, 2)              # [Hq, R, dh]
    sc = 1.0 / math.sqrt(q.shape[-1])
    s = np.matmul(qh, Kh.transpose(0, 2, 1)) * sc                      # [Hq, R, n]
    ds = (np.matmul(np.abs(qh), dKh.transpose(0, 2, 1)) + np.matmul(dqh, np.abs(Kh).transpose(0, 2, 1))) * sc
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    o = np.matmul(p, Vh)                                               # [Hq, R, dh]
    # d(sum_j p_j v_j) = sum_j p_j (ds_j - sum_k p_k ds_k) v_j + p_j dv_j  <=  sum_j p_j ds_j (|v_j| + |o|) + p dv
    pds = p * ds
    do = np.matmul(pds, np.abs(Vh)) + pds.sum(-1, keepdims=True) * np.abs(o) + np.matmul(p, dVh)
    dkl = None
    if P_prev is not None:
        pp = np.asarray(P_prev, np.float64).transpose(1, 0, 2)
        lq = pp - pp.max(-1, keepdims=True)
        lq = lq - np.log(np.exp(lq).sum(-1, keepdims=True))
        ls = np.log(np.maximum(p, 1e-300))
        kl = np.sum(p * (ls - lq), axis=-1, keepdims=True)
        # dKL/ds_j = p_j (ls_j - lq_j - KL); the softmax's own shift is covered by the sum of |.|
        dkl = np.sum(p * np.abs(ls - lq - kl) * ds, axis=-1).T          # [R, Hq]
    return ds.transpose(1, 0, 2), do.transpose(1, 0, 2), dkl


def swiglu_out_dev(hp, dhp, wg, wu, wd, eps):
    """Deviation of out = h' + (silu(g) * u) W_d^T, g/u = RMSNorm(h') W_g^T / W_u^T, for h'
    deviations dhp, to first order with absolute values throughout."""
    hp = np.asarray(hp, np.float64)
    b = hp / np.sqrt(np.mean(hp * hp, axis=-1, keepdims=True) + eps)
    db = rms_dev(hp, dhp, eps)
    g, u = b @ np.asarray(wg, np.float64).T, b @ np.asarray(wu, np.float64).T
    dg, du = proj_dev(db, wg), proj_dev(db, wu)
    sg = 1.0 / (1.0 + np.exp(-g))
    dsilu = sg * (1.0 + g * (1.0 - sg))
    dact = np.abs(dsilu * u) * dg + np.abs(g * sg) * du
    return np.abs(dhp) + proj_dev(dact, wd)


def explained(a, b, allow, rtol=2e-3, floor=1e-3):
    """Elementwise check |a - b| <= rtol max(|b|, floor max|b|) + SAFETY * allow.  Returns
    (ok mask, number of elements inside the bound only thanks to the allowance)."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    tol = rtol * np.maximum(np.abs(b), floor * np.abs(b).max()) if b.size else 0.0
    err = np.abs(a - b)
    ok = err <= tol + SAFETY * np.asarray(allow, np.float64)
    return ok, int(np.sum(ok & (err > tol)))


def drift_call_allow(O, cfg, W, blk_start, h_act, h_win, patched, Z, K_after, V_after, proxy_q, proxy_keys,
                     P_prev, act_prev=None, refresh=True):
    """Allowances of one polestar_drift call's outputs (oracle values only).

    The call projects round(RMSNorm(.)) of [active; window; centroids] rows, stores the K/V rows
    of the active block and of the patched window rows, and attends over the cache it has just
    written.  Arguments are the oracle's inputs of the call and its cache after the call.
    Returns {"qkv", "o", "act_logits", "proxy_logits", "delta", "D"} (missing when not
    computed by the call)."""
    st, eps, dt = cfg.st, cfg.eps, cfg.dtype
    B, hq, hkv, dh, n = cfg.B, cfg.hq, cfg.hkv, cfg.dh, cfg.n
    nq, nkv = hq * dh, hkv * dh
    wqkv = np.concatenate([W["wq"], W["wk"], W["wv"]], 0)
    toks = np.concatenate([h_act, h_win], 0) if refresh else np.asarray(h_act)
    rows_all = np.concatenate([toks, Z], 0) if refresh else toks
    proj = O.project(rows_all, wqkv, eps, st)
    dproj = proj_dev(norm_in_dev(rows_all, eps, dt), wqkv)
    wpos = O.window_positions(blk_start, n, B, cfg.pre, cfg.suf)
    patched = np.zeros(len(wpos), dtype=bool) if (patched is None or not refresh) else np.asarray(patched)
    written = np.concatenate([np.arange(B), B + np.nonzero(patched)[0]])
    pos_w = np.concatenate([np.arange(blk_start, blk_start + B), wpos[patched]])
    dK, dV = np.zeros((n, hkv, dh)), np.zeros((n, hkv, dh))
    dK[pos_w] = stored_dev(proj[written, nq:nq + nkv], dt, dproj[written, nq:nq + nkv]).reshape(-1, hkv, dh)
    dV[pos_w] = stored_dev(proj[written, nq + nkv:], dt, dproj[written, nq + nkv:]).reshape(-1, hkv, dh)
    nt = len(toks)
    q_tok = proj[:nt, :nq].reshape(-1, hq, dh)
    dq_tok = dproj[:nt, :nq].reshape(-1, hq, dh)
    dlg, do, _ = attn_dev(q_tok, K_after, V_after, dq_tok, dK, dV, hq, hkv)
    out = {"qkv": dproj, "o": do.reshape(nt, nq), "act_logits": dlg[:B]}
    if act_prev is not None:
        out["delta"] = attn_dev(q_tok[:B], K_after, V_after, dq_tok[:B], dK, dV, hq, hkv, P_prev=act_prev)[2].sum(-1)
    if refresh:
        dlp, _, dkl = attn_dev(proxy_q, K_after, V_after, dproj[nt:, :nq].reshape(-1, hq, dh), dK, dV, hq, hkv,
                               P_prev=np.asarray(P_prev)[..., proxy_keys], keys=proxy_keys)
        out["proxy_logits"] = dlp
        out["D"] = dkl.sum(-1)
    return out


def refresh_call_allow(O, cfg, W, rf, o_allow, S, wkv_next=None):
    """Allowances of one polestar_refresh call's outputs: h', the layer outputs (before their
    rounding) of rows [active; S], and (wkv_next given) the next layer's K/V projections of the
    update packet, which this call stores and projects again.  o_allow: the attention-output
    allowance rows [active; window] of the drift call."""
    B = cfg.B
    S = np.asarray(S, dtype=np.int64)
    do_rows = np.concatenate([o_allow[:B], o_allow[B + S]], 0)
    dhp = proj_dev(do_rows, W["wo"])
    dout = swiglu_out_dev(rf["hp"], dhp, W["wg"], W["wu"], W["wd"], cfg.eps)
    out = {"hp": dhp, "out": dout}
    if wkv_next is not None:
        dU = stored_dev(rf["out_pre"][B:], cfg.dtype, dout[B:])
        out["kv"] = proj_dev(norm_in_dev(rf["U"], cfg.eps, cfg.dtype, dU), wkv_next)
    return out
