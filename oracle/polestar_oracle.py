"""CPU oracle for Polestar-Cache's drift-scored sparse KV refresh and Polestar-Commit.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never calls it, and this module imports nothing from it.

Source: "Polestar: Drift-Aware Cache Calibration and Token Commitment for
Efficient Inference of Diffusion LLMs" (arXiv 2607.14107).  Citations below
name that page's sections, equations, tables and Algorithm 1.

Everything is plain NumPy in float64.  The method is a heuristic iteration, so
the oracle follows its steps in the page's order.  The page's full-precision
baseline is a 16-bit model (Table 11) and it does not say where values are
rounded.  The oracle rounds (``st`` = round to the storage dtype, identity for
"f64") at exactly these points:
  * tensors that outlive a call: the K/V cache, window rows, centroids (after
    normalisation), the layer outputs ``out = st(h' + act Wd^T)`` (active rows
    and update packet U); attention logits kept as the next step's reference
    are stored as float32;
  * the input of every projection of such a stored row, its RMSNorm output
    (unit gain, eps): ``st(x / rms(x))`` for the QKV and proxy-query
    projections of hidden rows and centroids, the next layer's K/V of U and the
    LM head;
  * the NVFP4 codec and the commit rule are evaluated in float32, the
    precision in which the GPU takes those integer decisions.
Values produced and consumed inside one call stay unrounded: the queries, the
attention output ``o``, ``h' = h + o Wo^T``, RMSNorm(h') and the SwiGLU
product ``act``.  (Rounding them too would chain five roundings inside one
refresh call; each turns a deviation of relative size e between two correct
implementations into one of about sqrt(e * 2^-8), which ends near 2e-3.)
Softmax, log-sum-exp, KL and every accumulation stay in float64.
Functions that only the mathematics pins are marked in their docstrings.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------


def round_bf16(x) -> np.ndarray:
    """Round float64 values once to bfloat16 (8 significant bits), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, |m| in [0.5, 1)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # np.rint is round-half-even
    return np.where(np.isfinite(x), r, x)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def storer(dtype: str):
    """Rounding applied where the GPU path stores a value in its storage dtype."""
    if dtype == "bf16":
        return round_bf16
    if dtype == "f32":
        return round_f32
    if dtype == "f64":
        return lambda x: np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# positions: active block and local window  [Polestar §2 "KV Caching in dLLMs";
# §4.1 "Block entry"; §5.1 hyper-parameters: |Omega_p| = 2B, |Omega_s| = B]
# ---------------------------------------------------------------------------


def active_positions(blk_start: int, B: int) -> np.ndarray:
    return np.arange(blk_start, blk_start + B, dtype=np.int64)


def window_positions(blk_start: int, n: int, B: int, pre: int, suf: int) -> np.ndarray:
    """Prefix window before the active block plus suffix window after it.

    The active block itself is not part of the window (it is recomputed at
    every step); both sides are truncated at the sequence ends.
    """
    prefix = list(range(max(0, blk_start - pre), blk_start))
    suffix = list(range(blk_start + B, min(n, blk_start + B + suf)))
    return np.asarray(prefix + suffix, dtype=np.int64)


def suffix_mask(blk_start: int, n: int, B: int, pre: int, suf: int) -> np.ndarray:
    pos = window_positions(blk_start, n, B, pre, suf)
    return pos >= blk_start + B


# ---------------------------------------------------------------------------
# layer pieces  [Polestar App. B "setup": logits q.k / sqrt(d_h), softmax,
# output sum_j a_j v_j; pre-norm transformer with RMSNorm and SwiGLU]
# ---------------------------------------------------------------------------


def rms(x: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return np.sqrt(np.mean(x * x, axis=-1) + eps)


def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    return np.asarray(x, dtype=np.float64) / rms(x, eps)[..., None]


def norm_in(x: np.ndarray, eps: float, st=None) -> np.ndarray:
    """RMSNorm output (unit gain) as a projection input, rounded by ``st`` when given."""
    a = rmsnorm(x, eps)
    return a if st is None else st(a)


def project(x: np.ndarray, w: np.ndarray, eps: float, st=None) -> np.ndarray:
    """RMSNorm(x) @ W^T with unit gain; ``st`` rounds the normalised rows first."""
    return norm_in(x, eps, st) @ np.asarray(w, dtype=np.float64).T


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def logsumexp(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))[..., 0]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int, n_kv: int):
    """Softmax attention of query rows over every key position.

    q: [R, Hq, dh]; k, v: [n, Hkv, dh].  Query head h reads KV head
    floor(h * Hkv / Hq) (grouped-query sharing).  Returns (out [R, Hq, dh],
    logits [R, Hq, n]).
    """
    R, hq, dh = q.shape
    assert hq == n_heads
    g = (np.arange(n_heads) * n_kv) // n_heads
    kk = np.asarray(k, dtype=np.float64)[:, g, :].transpose(1, 2, 0)      # [Hq, dh, n]
    vv = np.asarray(v, dtype=np.float64)[:, g, :].transpose(1, 0, 2)      # [Hq, n, dh]
    qh = np.asarray(q, dtype=np.float64).transpose(1, 0, 2)               # [Hq, R, dh]
    logits = np.matmul(qh, kk) / math.sqrt(dh)                            # [Hq, R, n]
    p = np.exp(logits - logsumexp(logits)[..., None])
    out = np.matmul(p, vv)                                                # [Hq, R, dh]
    return out.transpose(1, 0, 2), logits.transpose(1, 0, 2)


# ---------------------------------------------------------------------------
# drift  [Polestar Eq. 4: D = KL(A_t || A_{t-1}) between attention
# distributions of consecutive steps; §4.1 proxy attention of centroids]
# ---------------------------------------------------------------------------


def kl_logits(s: np.ndarray, s_prev: np.ndarray) -> np.ndarray:
    """KL(softmax(s) || softmax(s_prev)) along the last axis, natural log.

    Plain definition: sum_j p_j (log p_j - log p'_j) with p = softmax(s).
    """
    s = np.asarray(s, dtype=np.float64)
    s_prev = np.asarray(s_prev, dtype=np.float64)
    logp = s - logsumexp(s)[..., None]
    logq = s_prev - logsumexp(s_prev)[..., None]
    return np.sum(np.exp(logp) * (logp - logq), axis=-1)


def head_summed_drift(s: np.ndarray, s_prev: np.ndarray) -> np.ndarray:
    """Per row: sum over heads of max(0, KL) (heads on axis -2, keys on -1)."""
    return np.sum(np.maximum(kl_logits(s, s_prev), 0.0), axis=-1)


# ---------------------------------------------------------------------------
# spherical k-means  [Polestar §4.1 "Cluster and Quantize Hidden States";
# Algorithm 1 block-entry clustering; K = 8 (§5.1, Table 5)]
# ---------------------------------------------------------------------------


def unit_rows(h: np.ndarray) -> np.ndarray:
    h = np.asarray(h, dtype=np.float64)
    nrm = np.sqrt(np.sum(h * h, axis=-1))
    out = np.zeros_like(h)
    nz = nrm > 0
    out[nz] = h[nz] / nrm[nz, None]
    return out


def spherical_kmeans(h: np.ndarray, n_clusters: int, init_idx: np.ndarray, iters: int = 10):
    """Lloyd iterations of spherical k-means on the rows of ``h``.

    Rows are projected to the unit sphere; centroids start at the rows named by
    ``init_idx`` (min(K, rows) of them).  Each iteration assigns every row to
    the centroid of largest cosine (lowest index on ties) and then sets every
    non-empty cluster's centroid to the normalised sum of its members (an
    empty cluster keeps its centroid).  Returns (Z [K, d] float64 unit rows,
    zero rows for clusters beyond min(K, rows), M [rows] int, trace [2*iters])
    where the trace holds the objective sum_i x_i . z_M(i) after every
    assignment and after every update.
    """
    x = unit_rows(h)
    nw, d = x.shape
    k_eff = min(n_clusters, nw)
    init_idx = np.asarray(init_idx, dtype=np.int64)
    assert len(init_idx) == k_eff and len(set(init_idx.tolist())) == k_eff
    z = np.zeros((n_clusters, d))
    z[:k_eff] = x[init_idx]
    m = np.zeros(nw, dtype=np.int64)
    trace = []
    for _ in range(iters):
        cos = x @ z[:k_eff].T                        # [nw, k_eff]
        m = np.argmax(cos, axis=1)                   # first maximum = lowest index
        trace.append(float(np.sum(cos[np.arange(nw), m])))
        for c in range(k_eff):
            mem = m == c
            if mem.any():
                s = np.sum(x[mem], axis=0)
                ns = np.sqrt(np.sum(s * s))
                if ns > 0:
                    z[c] = s / ns
        trace.append(float(np.sum(x * z[m])))
    return z, m.astype(np.int32), np.asarray(trace)


def centroid_update(h: np.ndarray, m: np.ndarray, z_old: np.ndarray) -> np.ndarray:
    """Incremental centroid refresh with the labels held fixed [§4.1].

    One spherical k-means update step on the current (patched) window rows:
    z_c = normalise(sum of member unit rows); empty clusters keep z_old.
    """
    x = unit_rows(h)
    z = np.array(z_old, dtype=np.float64, copy=True)
    for c in range(z.shape[0]):
        mem = np.asarray(m) == c
        if mem.any():
            s = np.sum(x[mem], axis=0)
            ns = np.sqrt(np.sum(s * s))
            if ns > 0:
                z[c] = s / ns
    return z


# ---------------------------------------------------------------------------
# NVFP4 residual storage  [Polestar App. C.3: 1 sign, 2 exponent, 1 mantissa
# bit per value, FP8 E4M3 scale per group of 16; §4.1 residual to centroid;
# Table 11 "residual NVFP4"]
# ---------------------------------------------------------------------------

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_value(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAG[code & 7]
    return np.where(code & 8, -mag, mag)


def e4m3_value(code) -> np.ndarray:
    """OCP E4M3FN: bias 7, subnormal step 2^-9, max 448, 0x7F/0xFF are NaN."""
    code = np.asarray(code, dtype=np.int64)
    e = (code >> 3) & 0xF
    mt = code & 7
    mag = np.where(e == 0, mt * 2.0 ** -9, np.ldexp(1.0 + mt / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return np.where(code & 0x80, -mag, mag)


_E4M3_POS = e4m3_value(np.arange(0x7F))            # 127 finite non-negative values


def _nearest_even(x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest table value; on an exact tie the even index wins."""
    dist = np.abs(x[..., None] - table)
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    even = cand & ((np.arange(len(table)) & 1) == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return pick


def e4m3_encode(x) -> np.ndarray:
    """Round non-negative values to E4M3FN, nearest with ties to even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(x >= 0)
    x = np.minimum(x, 448.0)
    return _nearest_even(x, _E4M3_POS).astype(np.uint8)


def e2m1_encode(y) -> np.ndarray:
    """Round to E2M1, nearest with ties to even code, saturating at +-6; zero is +0."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), 6.0)
    c = _nearest_even(mag, E2M1_MAG).astype(np.int64)
    neg = (y < 0) & (c != 0)
    return (c | np.where(neg, 8, 0)).astype(np.uint8)


def nvfp4_quantize(r: np.ndarray):
    """Quantise float32 rows [rows, d] to (codes [rows, d/2] u8, scales [rows, d/16] u8).

    Per group of 16 consecutive channels: s = amax / 6 (float32 division),
    scale byte = E4M3(s); s' = its value; if s' == 0 every code is 0, else
    code = E2M1(r / s') (float32 division).  Element 2j goes in the low nibble.
    """
    r = np.asarray(r, dtype=np.float32)
    rows, d = r.shape
    assert d % 16 == 0
    g = r.reshape(rows, d // 16, 16)
    amax = np.max(np.abs(g), axis=-1)
    s = (amax.astype(np.float32) / np.float32(6.0)).astype(np.float32)
    sc = e4m3_encode(s.astype(np.float64))
    sv = e4m3_value(sc).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (g / sv[..., None]).astype(np.float32)
    codes = np.where(sv[..., None] == 0, 0, e2m1_encode(np.where(sv[..., None] == 0, 0.0, y))).astype(np.uint8)
    codes = codes.reshape(rows, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc.astype(np.uint8)


def nvfp4_dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, half * 2), dtype=np.int64)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    vals = e2m1_value(codes).reshape(rows, half * 2 // 16, 16)
    sv = e4m3_value(scales.astype(np.int64))
    return (vals * sv[..., None]).reshape(rows, half * 2).astype(np.float32)


# ---------------------------------------------------------------------------
# Other residual formats  [Polestar Table 11 ablation: FP8, INT8, MXFP4 residuals.
# The pages name the formats only; readings: FP8 = OCP E4M3FN per value, no scale;
# INT8 and MXFP4 = OCP microscaling blocks of 32 values sharing one E8M0
# (power-of-two) scale, X = 2^(floor(log2 amax) - emax), emax = 0 for INT8
# (values q * 2^-6, q in [-128, 127]) and 2 for E2M1 (MXFP4).]
# ---------------------------------------------------------------------------


def fp8_quantize(r: np.ndarray):
    """Residual rows [rows, d] -> E4M3FN bytes [rows, d] (sign bit | magnitude code, nearest
    even, saturating at 448; zero is +0).  No scales."""
    r = np.asarray(r, dtype=np.float32)
    mag = e4m3_encode(np.abs(r).astype(np.float64)).astype(np.uint8)
    neg = (r < 0) & (mag != 0)
    return (mag | np.where(neg, 0x80, 0)).astype(np.uint8), np.zeros((r.shape[0], 0), dtype=np.uint8)


def fp8_dequantize(codes: np.ndarray, scales=None) -> np.ndarray:
    return e4m3_value(np.asarray(codes, dtype=np.int64)).astype(np.float32)


def mx_exponent(amax: np.ndarray, emax: int) -> np.ndarray:
    """Shared E8M0 exponent of a block: floor(log2(amax)) - emax, clamped to [-127, 127];
    -127 for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = f * 2^e, f in [0.5, 1)
    x = np.where(amax > 0, e - 1 - emax, -127)
    return np.clip(x, -127, 127).astype(np.int64)


def mxint8_quantize(r: np.ndarray):
    """Rows [rows, d] -> (int8 codes as u8 [rows, d], E8M0 scale bytes [rows, d/32]).

    Per block of 32: X = 2^(floor(log2 amax)); q = clamp(rne(r / X * 64), -128, 127).
    """
    r = np.asarray(r, dtype=np.float32)
    rows, d = r.shape
    assert d % 32 == 0
    g = r.reshape(rows, d // 32, 32).astype(np.float64)
    ex = mx_exponent(np.max(np.abs(g), axis=-1), 0)
    y = np.ldexp(g, (6 - ex)[..., None])                 # exact: r / X * 2^6
    q = np.clip(np.rint(y), -128, 127).astype(np.int64)  # np.rint: nearest, ties to even
    return (q & 0xFF).astype(np.uint8).reshape(rows, d), (ex + 127).astype(np.uint8)


def mxint8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    q = np.where(c >= 128, c - 256, c)
    rows, d = q.shape
    ex = np.asarray(scales, dtype=np.int64) - 127
    v = np.ldexp(q.reshape(rows, d // 32, 32).astype(np.float64), (ex - 6)[..., None])
    return v.reshape(rows, d).astype(np.float32)


def mxfp4_quantize(r: np.ndarray):
    """Rows [rows, d] -> (E2M1 nibbles packed [rows, d/2], E8M0 scale bytes [rows, d/32]).

    Per block of 32: X = 2^(floor(log2 amax) - 2); code = E2M1(r / X) (nearest even,
    saturating at 6).  Element 2j goes in the low nibble.
    """
    r = np.asarray(r, dtype=np.float32)
    rows, d = r.shape
    assert d % 32 == 0
    g = r.reshape(rows, d // 32, 32).astype(np.float64)
    ex = mx_exponent(np.max(np.abs(g), axis=-1), 2)
    codes = e2m1_encode(np.ldexp(g, (-ex)[..., None])).astype(np.uint8).reshape(rows, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (ex + 127).astype(np.uint8)


def mxfp4_dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, half * 2), dtype=np.int64)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    ex = np.asarray(scales, dtype=np.int64) - 127
    v = np.ldexp(e2m1_value(codes).reshape(rows, half * 2 // 32, 32), ex[..., None])
    return v.reshape(rows, half * 2).astype(np.float32)


RESID_CODECS = {
    "nvfp4": (nvfp4_quantize, nvfp4_dequantize),
    "fp8": (fp8_quantize, fp8_dequantize),
    "mxint8": (mxint8_quantize, mxint8_dequantize),
    "mxfp4": (mxfp4_quantize, mxfp4_dequantize),
}


def residual_quantize(h: np.ndarray, z: np.ndarray, m: np.ndarray, fmt: str = "nvfp4"):
    """Codes of r = float32(h) - float32(z_M(i)) (one float32 subtraction) in format fmt."""
    r = (np.asarray(h, dtype=np.float32) - np.asarray(z, dtype=np.float32)[np.asarray(m)]).astype(np.float32)
    return RESID_CODECS[fmt][0](r)


def residual_dequantize(packed, scales, z, m, st, fmt: str = "nvfp4") -> np.ndarray:
    """Window rows rebuilt as st(float32(z_M(i)) + dequant(r)) (float32 add, then store)."""
    base = np.asarray(z, dtype=np.float32)[np.asarray(m)]
    s = (base + RESID_CODECS[fmt][1](packed, scales)).astype(np.float32)
    return st(s.astype(np.float64))


# ---------------------------------------------------------------------------
# KV-cache staleness and selection accuracy  [Polestar App. C.2: E_i = 1 - mean of
# the K and V cosine similarities between cached and recomputed rows, each averaged
# over heads; §3 / Fig. 6(a): accuracy of a policy's top-25% positions against the
# true top-25% most stale positions]
# ---------------------------------------------------------------------------


def cosine(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine similarity along the last axis; 0 where either vector is zero (reading)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    na, nb = np.linalg.norm(a, axis=-1), np.linalg.norm(b, axis=-1)
    dot = np.sum(a * b, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where((na > 0) & (nb > 0), dot / (na * nb), 0.0)


def kv_staleness(k: np.ndarray, v: np.ndarray, k_ref: np.ndarray, v_ref: np.ndarray) -> np.ndarray:
    """E_i for every position of caches [n, H, dh] against recomputed [n, H, dh]."""
    ck = np.mean(cosine(k, k_ref), axis=-1)
    cv = np.mean(cosine(v, v_ref), axis=-1)
    return 1.0 - 0.5 * (ck + cv)


def top_fraction(scores: np.ndarray, frac: float) -> np.ndarray:
    """Indices of the ceil(frac * n) largest scores; equal scores -> lower index first."""
    scores = np.asarray(scores, dtype=np.float64)
    m = int(math.ceil(frac * len(scores)))
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    return np.asarray(sorted(order[:m]), dtype=np.int64)


def attended_token_change(q: np.ndarray, K_now: np.ndarray, K_ref: np.ndarray, hq: int, hkv: int):
    """The most-attended-token cosine policy that the drift ablation compares with [§5
    "Drift Measurement Policy", Fig. 6(a): each candidate position is ranked by the cosine
    change of its most-attended token].

    q [rows, hq, dh] are the candidate positions' queries, K_now [n, hkv, dh] the cache they
    attend over, K_ref [n, hkv, dh] the keys it is compared with.  Reading: a position's
    most-attended token j* is the argmax over positions of the attention probability averaged
    over the query heads (query head h reads KV head h * hkv // hq; lowest position on ties), and
    its change is 1 - the mean over KV heads of cos(K_now[j*], K_ref[j*]) (0 for a zero row).
    Returns (j_star [rows], score [rows], A [rows, n] head-mean probabilities).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K_now, dtype=np.float64)
    Kr = np.asarray(K_ref, dtype=np.float64)
    dh = q.shape[-1]
    g = (np.arange(hq) * hkv) // hq
    logits = np.einsum("rhd,jhd->rhj", q, K[:, g, :]) / math.sqrt(dh)
    p = np.exp(logits - logsumexp(logits)[..., None])
    A = p.mean(axis=1)
    j_star = np.argmax(A, axis=1)               # first maximum: the lowest position
    score = 1.0 - np.mean(cosine(K[j_star], Kr[j_star]), axis=-1)
    return j_star.astype(np.int64), score, A


def selection_accuracy(chosen, stale: np.ndarray, frac: float = 0.25) -> float:
    """Share of the true top-frac most stale positions that a policy's choice contains."""
    truth = set(int(i) for i in top_fraction(stale, frac))
    return len(truth & set(int(i) for i in chosen)) / max(len(truth), 1)


# ---------------------------------------------------------------------------
# selection  [§4.1 top-k clusters by drift; Algorithm 1 TopK and S = M[K]]
# ---------------------------------------------------------------------------


def topk_clusters(D: np.ndarray, k: int, k_eff: Optional[int] = None) -> np.ndarray:
    """The k clusters of largest drift among the first k_eff; equal drift -> lower index."""
    D = np.asarray(D)
    k_eff = len(D) if k_eff is None else k_eff
    order = sorted(range(k_eff), key=lambda c: (-float(D[c]), c))
    return np.asarray(order[: min(k, k_eff)], dtype=np.int32)


def select_rows(m: np.ndarray, topk: np.ndarray) -> np.ndarray:
    """Window rows (ascending) whose cluster is one of the selected clusters."""
    chosen = set(int(c) for c in topk)
    return np.asarray([i for i, c in enumerate(np.asarray(m)) if int(c) in chosen], dtype=np.int32)


# ---------------------------------------------------------------------------
# update schedule  [§4.1 "Update Schedule"; tau_upd = 3 (§5.1)]
# ---------------------------------------------------------------------------


def should_refresh(decoded_since_refresh: int, tau_upd: Optional[int]) -> bool:
    """Refresh once the tokens decoded since the last refresh exceed tau_upd (None = never)."""
    if tau_upd is None:
        return False
    return decoded_since_refresh > tau_upd


# ---------------------------------------------------------------------------
# one refresh step of one layer  [§4.1 "Measuring Drift and Layer-wise KV
# Updates"; Algorithm 1 in-block loop]
# ---------------------------------------------------------------------------


class Cfg:
    """Shapes and hyper-parameters the oracle needs (mirrors the workload recipe)."""

    def __init__(self, d, n_heads, n_kv_heads, head_dim, ffn, n_pos, block, win_prefix, win_suffix,
                 n_clusters, top_k, dtype, resid="raw", rms_eps=1e-6, hist=5, alpha=10.0,
                 tau_s=0.9, tau_suf=0.9, kmeans_iters=10, proxy_support="all", **_):
        self.d, self.hq, self.hkv, self.dh, self.ffn = d, n_heads, n_kv_heads, head_dim, ffn
        self.n, self.B, self.pre, self.suf = n_pos, block, win_prefix, win_suffix
        self.K, self.k = n_clusters, top_k
        self.dtype, self.resid, self.eps = dtype, resid, rms_eps
        self.hist, self.alpha, self.tau_s, self.tau_suf = hist, alpha, tau_s, tau_suf
        self.iters = kmeans_iters
        assert proxy_support in ("all", "active")
        self.proxy_support = proxy_support
        self.st = storer(dtype)

    @staticmethod
    def from_workload(w, dtype=None, **over):
        kw = dict(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn,
                  n_pos=w.n_pos, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix,
                  n_clusters=w.n_clusters, top_k=w.top_k, dtype=dtype or w.dtype, resid=w.resid,
                  rms_eps=w.rms_eps, hist=w.hist, alpha=w.alpha, tau_s=w.tau_s, tau_suf=w.tau_suf,
                  kmeans_iters=w.kmeans_iters, proxy_support=getattr(w, "proxy_support", "all"))
        kw.update(over)
        return Cfg(**kw)


def proxy_keys(cfg: Cfg, blk_start: int) -> np.ndarray:
    """Key positions of the proxy attention [§4.1 "Measuring Drift and Layer-wise KV Updates";
    Eq. 3].  "all": every position, the cached keys joined with the recomputed active-block keys
    (the support the drift of Eq. 4 is defined over); "active": the active block's keys only."""
    if cfg.proxy_support == "active":
        return active_positions(blk_start, cfg.B)
    return np.arange(cfg.n, dtype=np.int64)


def proxy_drift(zq: np.ndarray, K: np.ndarray, V: np.ndarray, P_prev: np.ndarray, cfg: Cfg, blk_start: int):
    """Proxy attention logits of the centroid queries over the proxy keys and their KL drift
    against the previous logits of the same keys (P_prev [K, Hq, n], logits at key positions).
    Returns (logits [K, Hq, len(keys)], kl [K, Hq], key positions)."""
    keys = proxy_keys(cfg, blk_start)
    _, plog = attention(zq, K[keys], V[keys], cfg.hq, cfg.hkv)
    return plog, kl_logits(plog, np.asarray(P_prev)[..., keys]), keys


def window_rows_now(ls: Dict, cfg: Cfg) -> np.ndarray:
    """Current window hidden rows: raw storage, or NVFP4 residual + centroid."""
    if cfg.resid != "raw":
        return residual_dequantize(ls["codes"], ls["scales"], ls["Z"], ls["M"], cfg.st, cfg.resid)
    return np.array(ls["H"], dtype=np.float64, copy=True)


def cluster_update(ls: Dict, cfg: Cfg, u_rows=None, u_idx=None) -> Dict:
    """Dequantise, patch with the incoming update packet, refresh centroids, re-quantise.

    [§4.1: the next layer refreshes its cached hidden states from the packet
    and updates the centroids incrementally; Algorithm 1 Dequantize / Patch /
    ResidualQuantization.]  Mutates ``ls`` (H or codes/scales, Z) and returns
    {"h": patched window rows, "patched": bool mask}.
    """
    h = window_rows_now(ls, cfg)
    patched = np.zeros(h.shape[0], dtype=bool)
    if u_idx is not None and len(u_idx):
        h[np.asarray(u_idx)] = np.asarray(u_rows, dtype=np.float64)
        patched[np.asarray(u_idx)] = True
    z_new = cfg.st(centroid_update(h, ls["M"], ls["Z"]))
    ls["Z"] = z_new
    if cfg.resid != "raw":
        ls["codes"], ls["scales"] = residual_quantize(h, z_new, ls["M"], cfg.resid)
    else:
        ls["H"] = h.copy()
    return {"h": h, "patched": patched}


def drift_layer(ls: Dict, W: Dict, cfg: Cfg, blk_start: int, h_act: np.ndarray, h_win: np.ndarray,
                patched: np.ndarray, refresh: bool = True, commit_prev: Optional[np.ndarray] = None):
    """Main forward of the active block up to attention, proxy attention, drift, top-k, S.

    [§2 Eq. 3: active-block queries attend to cached KV joined with the
    recomputed active-block KV; §4.1 proxy attention of the projected
    centroids over the same keys; Eq. 4 drift; top-k clusters and S.]
    Mutates the layer's K/V cache (active rows and patched window rows) and its
    stored proxy logits.  Returns a dict of outputs.
    """
    st, eps = cfg.st, cfg.eps
    jpos = active_positions(blk_start, cfg.B)
    wpos = window_positions(blk_start, cfg.n, cfg.B, cfg.pre, cfg.suf)
    nw = len(wpos)
    hq, hkv, dh = cfg.hq, cfg.hkv, cfg.dh
    toks = np.concatenate([h_act, h_win], axis=0) if refresh else np.asarray(h_act)
    q = project(toks, W["wq"], eps, st).reshape(-1, hq, dh)
    kr = st(project(toks, W["wk"], eps, st)).reshape(-1, hkv, dh)
    vr = st(project(toks, W["wv"], eps, st)).reshape(-1, hkv, dh)
    K, V = ls["K"], ls["V"]
    K[jpos], V[jpos] = kr[: cfg.B], vr[: cfg.B]
    if refresh and patched is not None and patched.any():
        rows = np.nonzero(patched)[0]
        K[wpos[rows]] = kr[cfg.B + rows]
        V[wpos[rows]] = vr[cfg.B + rows]
    out, logits = attention(q, K, V, hq, hkv)
    res = {"o": out.reshape(out.shape[0], hq * dh), "q": q,
           "act_logits": round_f32(logits[: cfg.B])}
    if commit_prev is not None:
        res["delta"] = head_summed_drift(logits[: cfg.B], commit_prev)
    if refresh:
        k_eff = min(cfg.K, nw)
        zq = project(ls["Z"], W["wq"], eps, st).reshape(cfg.K, hq, dh)
        plog, kl, keys = proxy_drift(zq, K, V, ls["P"], cfg, blk_start)   # kl: [K, Hq]
        D = np.sum(np.maximum(kl, 0.0), axis=1)
        D[k_eff:] = 0.0
        topk = topk_clusters(D, cfg.k, k_eff)
        S = select_rows(ls["M"], topk)
        P = np.array(ls["P"], dtype=np.float64, copy=True)
        P[..., keys] = round_f32(plog)
        ls["P"] = P
        res.update(D=D, kl=kl, topk=topk, S=S, proxy_q=zq, proxy_logits=plog, proxy_keys=keys)
    return res


def refresh_layer(W: Dict, cfg: Cfg, h_act: np.ndarray, h_win: np.ndarray, o_tok: np.ndarray,
                  S: np.ndarray):
    """Gathered sparse forward over the active block and the selected rows S.

    [§4.1: layer forward only over the hidden states of the top-k clusters;
    its outputs form the update packet for layer l+1.]  Rows are
    [active block; S].  Returns the stored outputs (h_act_out, U), the
    layer output before its rounding (out_pre) and the unrounded h' and SwiGLU
    product.
    """
    st, eps, B = cfg.st, cfg.eps, cfg.B
    S = np.asarray(S, dtype=np.int64)
    x = np.concatenate([h_act, h_win[S]], axis=0)
    o = np.concatenate([o_tok[:B], o_tok[B + S]], axis=0)
    hp = x + o @ np.asarray(W["wo"], dtype=np.float64).T
    g = project(hp, W["wg"], eps)
    u = project(hp, W["wu"], eps)
    act = silu(g) * u
    out_pre = hp + act @ np.asarray(W["wd"], dtype=np.float64).T
    out = st(out_pre)
    return {"h_act_out": out[:B], "U": out[B:], "out_pre": out_pre, "hp": hp, "act": act}


def kv_rows(u: np.ndarray, wk: np.ndarray, wv: np.ndarray, cfg: Cfg):
    """K/V of layer l+1 for the packet rows, from the fresh U [§4.1; Algorithm 1 Patch]."""
    k = cfg.st(project(u, wk, cfg.eps, cfg.st)).reshape(-1, cfg.hkv, cfg.dh)
    v = cfg.st(project(u, wv, cfg.eps, cfg.st)).reshape(-1, cfg.hkv, cfg.dh)
    return k, v


# ---------------------------------------------------------------------------
# Polestar-Commit  [§4.2 "Current Block Commit", "Suffix Block Commit";
# Table 5: tau_s = 0.9, h = 5, alpha = 10, suffix confidence 0.9]
# ---------------------------------------------------------------------------


def confidence(x: np.ndarray, w_lm: np.ndarray, mask_id: int, eps: float, st=None):
    """Softmax max-probability over the vocabulary excluding the mask token [§2 Eq. 1].

    Logits = st(RMSNorm(x)) @ W_lm^T (unit gain, the normalised rows rounded
    like every projection input); the softmax runs over every id;
    c = max over ids != mask_id, yhat = its argmax (lowest id on ties).
    """
    logits = project(x, w_lm, eps, st)
    c, yhat = confidence_from_logits(logits, mask_id)
    return c, yhat, logits


def confidence_from_logits(logits: np.ndarray, mask_id: int):
    """The softmax part of :func:`confidence` for given LM-head logits [rows, vocab]."""
    logits = np.asarray(logits, dtype=np.float64)
    lse = logsumexp(logits)
    lg = logits.copy()
    lg[:, mask_id] = -np.inf
    yhat = np.argmax(lg, axis=1)
    c = np.exp(lg[np.arange(len(lg)), yhat] - lse)
    return c, yhat.astype(np.int32)


def commit_decide(delta, conf, masked, hist_vals, hist_cnt, hist_len, alpha, tau_s):
    """Current-block commit rule, evaluated in float32 in a fixed order.

    mean = (sum of the stored history values, oldest first) / count, 0 when
    empty; spike = delta - mean; tau_d = alpha * (tau_s - c)^2; commit when
    masked and (c >= tau_s or spike > tau_d).  The history then keeps the last
    ``hist_len`` values including this delta.  Returns (commit u8, spike f32,
    tau_d f32, new hist_vals, new hist_cnt).
    """
    f = np.float32
    delta = np.asarray(delta, dtype=np.float32)
    conf = np.asarray(conf, dtype=np.float32)
    nb = delta.shape[0]
    hv = np.array(hist_vals, dtype=np.float32, copy=True).reshape(nb, max(hist_len, 1))
    hc = np.array(hist_cnt, dtype=np.int32, copy=True)
    spike = np.zeros(nb, dtype=np.float32)
    taud = np.zeros(nb, dtype=np.float32)
    commit = np.zeros(nb, dtype=np.uint8)
    for j in range(nb):
        cnt = int(hc[j])
        if cnt > 0:
            acc = f(0.0)
            for i in range(cnt):
                acc = f(acc + hv[j, i])
            mean = f(acc / f(cnt))
        else:
            mean = f(0.0)
        spike[j] = f(delta[j] - mean)
        t = f(f(tau_s) - conf[j])
        taud[j] = f(f(alpha) * f(t * t))
        commit[j] = 1 if (masked[j] and (conf[j] >= f(tau_s) or spike[j] > taud[j])) else 0
        if hist_len > 0:
            if cnt < hist_len:
                hv[j, cnt] = delta[j]
                hc[j] = cnt + 1
            else:
                hv[j, :-1] = hv[j, 1:].copy()
                hv[j, -1] = delta[j]
    return commit, spike, taud, hv, hc


def entry_commit(conf, masked, tau):
    """Commit at block entry [§4.2; Algorithm 1 block entry]: there is no drift yet,
    so a masked row commits when its confidence reaches the threshold (tau_s for the
    active block, tau_suf for the suffix window), compared in float32."""
    conf = np.asarray(conf, dtype=np.float32)
    return (np.asarray(masked, dtype=bool) & (conf >= np.float32(tau))).astype(np.uint8)


def suffix_commit(conf, eligible, tau_suf):
    conf = np.asarray(conf, dtype=np.float32)
    return (np.asarray(eligible, dtype=bool) & (conf >= np.float32(tau_suf))).astype(np.uint8)


# ---------------------------------------------------------------------------
# full forward (block-entry state and the dense reference for the k = K pin)
# ---------------------------------------------------------------------------


def full_forward(h0: np.ndarray, layers: List[Dict], cfg: Cfg):
    """Dense forward of every position through every layer (bidirectional attention).

    Returns (H list of layer inputs incl. the final output [L+1][n, d],
    K list, V list, last-layer logits [n, Hq, n]).
    """
    st, eps = cfg.st, cfg.eps
    h = st(np.asarray(h0, dtype=np.float64))
    Hs, Ks, Vs = [h], [], []
    logits = None
    for W in layers:
        q = project(h, W["wq"], eps, st).reshape(-1, cfg.hq, cfg.dh)
        k = st(project(h, W["wk"], eps, st)).reshape(-1, cfg.hkv, cfg.dh)
        v = st(project(h, W["wv"], eps, st)).reshape(-1, cfg.hkv, cfg.dh)
        out, logits = attention(q, k, v, cfg.hq, cfg.hkv)
        o = out.reshape(out.shape[0], -1)
        hp = h + o @ np.asarray(W["wo"], dtype=np.float64).T
        act = silu(project(hp, W["wg"], eps)) * project(hp, W["wu"], eps)
        h = st(hp + act @ np.asarray(W["wd"], dtype=np.float64).T)
        Hs.append(h)
        Ks.append(k)
        Vs.append(v)
    return Hs, Ks, Vs, logits


def entry_positions(blk_start: int, n: int, B: int, pre: int, suf: int, full: bool) -> np.ndarray:
    """Positions whose hidden rows the block-entry forward recomputes.

    [§4.1 "Update Schedule": a forward of the whole sequence at every other
    block entry; Algorithm 1 block entry.]  Reading: a full entry covers every
    position; the other entries cover the window and the active block, the
    positions [blk_start - pre, blk_start + B + suf) cut at the sequence ends.
    """
    if full:
        return np.arange(n, dtype=np.int64)
    return np.arange(max(0, blk_start - pre), min(n, blk_start + B + suf), dtype=np.int64)


def layer_forward_rows(h_rows: np.ndarray, pos: np.ndarray, W: Dict, cfg: Cfg, K: np.ndarray, V: np.ndarray):
    """One layer's forward of the hidden rows at positions ``pos``.

    Their K/V replace the cache rows at ``pos`` first; every row then attends
    to all n cache positions (bidirectional), and the residual, RMSNorm and
    SwiGLU steps follow as in :func:`full_forward`.  Mutates K and V; returns
    the stored output rows.
    """
    st, eps = cfg.st, cfg.eps
    h = np.asarray(h_rows, dtype=np.float64)
    q = project(h, W["wq"], eps, st).reshape(-1, cfg.hq, cfg.dh)
    K[pos] = st(project(h, W["wk"], eps, st)).reshape(-1, cfg.hkv, cfg.dh)
    V[pos] = st(project(h, W["wv"], eps, st)).reshape(-1, cfg.hkv, cfg.dh)
    out, _ = attention(q, K, V, cfg.hq, cfg.hkv)
    hp = h + out.reshape(out.shape[0], -1) @ np.asarray(W["wo"], dtype=np.float64).T
    act = silu(project(hp, W["wg"], eps)) * project(hp, W["wu"], eps)
    return st(hp + act @ np.asarray(W["wd"], dtype=np.float64).T)


def block_entry_layer_state(H_in: np.ndarray, K: np.ndarray, V: np.ndarray, Wq: np.ndarray, cfg: Cfg,
                            blk_start: int, init_idx) -> Dict:
    """Cached state of one layer at block entry [§4.1 "Block entry"; Algorithm 1].

    Window hidden rows, spherical k-means centroids and labels, the residual
    codes (NVFP4) and the proxy logits that serve as the first drift reference.
    """
    wpos = window_positions(blk_start, cfg.n, cfg.B, cfg.pre, cfg.suf)
    hw = np.asarray(H_in, dtype=np.float64)[wpos]
    z, m, trace = spherical_kmeans(hw, cfg.K, init_idx, cfg.iters)
    z = cfg.st(z)
    ls = {"K": np.array(K, dtype=np.float64, copy=True), "V": np.array(V, dtype=np.float64, copy=True),
          "Z": z, "M": m, "trace": trace}
    if cfg.resid != "raw":
        ls["codes"], ls["scales"] = residual_quantize(hw, z, m, cfg.resid)
    else:
        ls["H"] = hw.copy()
    zq = project(z, Wq, cfg.eps, cfg.st).reshape(cfg.K, cfg.hq, cfg.dh)
    keys = proxy_keys(cfg, blk_start)
    _, plog = attention(zq, ls["K"][keys], ls["V"][keys], cfg.hq, cfg.hkv)
    ls["P"] = np.zeros((cfg.K, cfg.hq, cfg.n))
    ls["P"][..., keys] = round_f32(plog)
    return ls
