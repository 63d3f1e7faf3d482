"""Shared helpers of the GPU parity tests: device handle/workspace, identical
seeded state on both sides, and the comparison rules.

Inputs come from ``synth`` (generated on the GPU with the same integer
generator, then copied to the host for the oracle) or from the oracle itself;
nothing the HIP path computes is ever fed to the oracle.
"""
from __future__ import annotations

import math
import sys
from typing import Dict, Optional

import numpy as np
import torch

import synth
from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def to_dev(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload oracle values (exactly representable in ``dtype``)."""
    return torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64).to(TDT[dtype]).to(device)


# ---------------------------------------------------------------- comparisons
def _rows(x):
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(1, -1) if x.ndim <= 1 else x.reshape(-1, x.shape[-1])


def rel_err(a, b):
    """Elementwise |a - b| / max(|b|, RMS of b's row); rows are the last axis."""
    a2, b2 = _rows(a), _rows(b)
    if b2.size == 0:
        return np.zeros(0)
    rms = np.sqrt(np.mean(b2 * b2, axis=1, keepdims=True))
    return np.abs(a2 - b2) / np.maximum(np.maximum(np.abs(b2), rms), 1e-30)


def row_err(a, b):
    """Per row: ||a - b||_2 / ||b||_2."""
    a2, b2 = _rows(a), _rows(b)
    if b2.size == 0:
        return np.zeros(0)
    return np.linalg.norm(a2 - b2, axis=1) / np.maximum(np.linalg.norm(b2, axis=1), 1e-30)


# One bfloat16 ulp relative to a value's scale is at most 2^-7.  Storage-rounding
# decisions that the float32 GPU and the float64 oracle take differently at
# isolated near-midpoints move a stored element by one such ulp, and the elements
# computed from it by a few; rows as a whole stay within the 2e-3 bound.
BF16_ELEM_BOUND = 4 * 2.0 ** -8
FLOOR = 1e-3     # absolute floor of the per-call rule, as a fraction of the tensor's max |b|
# Attention logits are defined up to a shift of each row (the softmax does not see it), so their
# absolute error, set by the float32 accumulation of the 4096-long projections that produce the
# queries (about 1e-6 of |q||k|), is what matters; near zero it is judged against this floor.  The
# drift values the logits determine are held to FLOOR.
LOGIT_FLOOR = 1e-2


def rel_err_floor(a, b, floor=FLOOR):
    """Elementwise |a - b| / max(|b|, floor * max|b|), max|b| over the whole tensor."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b.size == 0:
        return np.zeros(b.shape)
    den = np.maximum(np.abs(b), floor * np.abs(b).max())
    return np.abs(a - b) / np.maximum(den, 1e-300)


def assert_close(a, b, name, rtol=2e-3, dtype="f32", allow=None, floor=FLOOR):
    """Per-call floating point (values before their storage rounding: projections, attention
    outputs, logits, drift, h', layer outputs): every element within rtol of the oracle's value,
    relative to max(|b|, floor max|b|) (floor 1e-3; logits LOGIT_FLOOR).  The floor keeps an element near zero from being judged
    against its own tiny magnitude.  ``allow`` (same shape, from tests.flips, computed from the
    oracle alone) adds the first-order effect of admissible alternative roundings of values
    stored earlier in the same call; the elements that need it are counted and reported.
    ``dtype`` only labels the log line."""
    from tests import flips as FL
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    e = rel_err_floor(a, b, floor)
    if e.size == 0:
        return 0.0
    r = row_err(a, b)
    al = np.zeros_like(b) if allow is None else np.broadcast_to(np.asarray(allow, np.float64), b.shape)
    ok, n_tie = FL.explained(a, b, al, rtol, floor)
    log(f"    {name}: max elem err {e.max():.2e} (floor {floor:g} max|b|), max row err {r.max():.2e}; "
        f"{n_tie} elements within the bound only through admissible tie roundings [{dtype}]")
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[int(np.argmax(e[tuple(bad.T)]))])
        raise AssertionError(f"{name}: {len(bad)} elements outside 2e-3 + tie allowance; worst at {i} of "
                             f"{b.shape}: got {a[i]!r}, want {b[i]!r}, allowance {al[i]:.3e}, rel err {e[i]:.3e}")
    return float(e.max())


def assert_derived(a, b, dtype, name, rtol=2e-3):
    """Values stored in the storage dtype, or computed from tensors that each side stored itself
    (so that inputs differ wherever a storage rounding went the other way): rows within rtol
    normwise; elements within rtol (float32) or a few bf16 ulps of their row's scale (bf16)."""
    e = rel_err(a, b)
    r = row_err(a, b)
    if e.size == 0:
        return 0.0
    el_bound = rtol if dtype == "f32" else max(rtol, BF16_ELEM_BOUND)
    i = int(np.argmax(e))
    log(f"    {name}: max row err {r.max():.2e}, max elem err {e.max():.2e} "
        f"(elems > {rtol:g}: {np.mean(e > rtol):.3%})")
    assert r.max() <= rtol, f"{name}: row error {r.max():.3e} > {rtol}"
    assert e.max() <= el_bound, (f"{name}: element error {e.max():.3e} > {el_bound:.3e} (flat idx {i}: "
                                 f"got {np.ravel(a)[i]!r}, want {np.ravel(b)[i]!r})")
    return float(r.max())


def assert_stored(a, b, dtype, name, rtol=2e-3):
    """Stored tensors (K/V cache, window rows, centroids, layer outputs): the bounds of
    assert_derived; also reports how many stored values differ at all, i.e. how many rounding
    decisions went the other way (for bf16: values one ulp apart)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    diff = int(np.sum(a != b)) if a.size else 0
    log(f"    {name}: {diff} of {a.size} stored values differ from the oracle's ({diff / max(a.size, 1):.3%})")
    assert_derived(a, b, dtype, name, rtol)
    return diff / max(a.size, 1)


def assert_rounded(stored, pre, dtype, name):
    """A stored tensor is its own pre-rounding value rounded once to the storage dtype.

    Floating-point parity is judged on the values before their storage rounding (a
    bf16 store alone moves a value by up to 2^-9 relative); this checks the store.
    """
    stored = np.asarray(stored, dtype=np.float64)
    want = O.storer(dtype)(np.asarray(pre, dtype=np.float64))
    bad = int(np.sum(stored != want))
    log(f"    {name}: stored = round(pre-rounding value) for {stored.size - bad}/{stored.size}")
    assert bad == 0, f"{name}: {bad} stored values are not the rounding of their pre-rounding value"


def assert_traj(a, b, dtype, name, rtol=2e-3):
    """Free-running values (each side continues from its own stored values; ``dtype`` is
    the storage dtype of the run): the tensor within rtol normwise; with bf16 storage
    every row within one bf16 ulp (2^-8) normwise and every element within a few ulps,
    with float32 storage both within rtol."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b.size == 0:
        return 0.0
    t = float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
    r, e = row_err(a, b), rel_err(a, b)
    row_bound = rtol if dtype == "f32" else 2.0 ** -8
    el_bound = rtol if dtype == "f32" else BF16_ELEM_BOUND
    log(f"    {name}: {float(np.mean(a != b)):.3%} values differ; tensor err {t:.2e}, max row err {r.max():.2e}, "
        f"max elem err {e.max():.2e}")
    assert t <= rtol, f"{name}: tensor error {t:.3e} > {rtol}"
    assert r.max() <= row_bound, f"{name}: row error {r.max():.3e} > {row_bound:.3e}"
    assert e.max() <= el_bound, f"{name}: element error {e.max():.3e} > {el_bound:.3e}"
    return t


def topk_margin(D, topk, k_eff):
    """Gap between the k-th selected and the best unselected drift (relative)."""
    D = np.asarray(D, dtype=np.float64)[:k_eff]
    sel = set(int(c) for c in topk if c >= 0)
    rest = [D[c] for c in range(k_eff) if c not in sel]
    if not rest or not sel:
        return np.inf
    lo = min(D[c] for c in sel)
    return (lo - max(rest)) / max(abs(lo), 1e-30)


TIE_REL = 1e-6   # drift values this close (relative) are a tie whichever implementation computes them


def check_topk(tg, Dg, D_or, topk_or, k, k_eff, tag, D_allow=None):
    """Top-k comparison.  The GPU's clusters must follow the rule on its own drift values; the
    selected set must equal the oracle's unless the oracle's gap between the k-th selected and
    the best unselected drift is within their admissible deviation (TIE_REL relative, plus
    SAFETY times D_allow, the oracle-derived effect of admissible tie roundings): then both sets
    are admissible, the near-tie is reported and False returned.  Within the set, the order may
    differ only between drifts tied in the same sense."""
    from tests import flips as FL
    kk = min(k, k_eff)
    tg = np.asarray(tg)[:kk]
    D_or = np.asarray(D_or, dtype=np.float64)
    al = np.zeros_like(D_or) if D_allow is None else np.asarray(D_allow, np.float64)
    tie = lambda x, y: abs(D_or[x] - D_or[y]) <= TIE_REL * max(abs(D_or[x]), abs(D_or[y])) + FL.SAFETY * (al[x] + al[y])
    assert np.array_equal(tg, O.topk_clusters(Dg, k, k_eff)[:kk]), f"{tag}: top-k does not follow the rule"
    sel_or = [int(c) for c in np.asarray(topk_or)[:kk]]
    if set(tg.tolist()) != set(sel_or):
        rest = [c for c in range(k_eff) if c not in sel_or]
        kth = min(sel_or, key=lambda c: (D_or[c], -c))
        best_rest = max(rest, key=lambda c: (D_or[c], -c))
        mg = topk_margin(D_or, topk_or, k_eff)
        if tie(kth, best_rest):
            log(f"    {tag}: top-k near-tie (oracle margin {mg:.2e}, clusters {kth}/{best_rest}), reported")
            return False
        raise AssertionError(f"{tag}: top-k {tg.tolist()} != oracle {sel_or} (margin {mg:.2e})")
    for a, b in zip(tg[:-1], tg[1:]):
        assert D_or[a] >= D_or[b] or tie(a, b), f"{tag}: top-k order {tg.tolist()} vs oracle drift"
    return True


# ---------------------------------------------------------------- device handle
class Dev:
    def __init__(self, w: synth.Workload, batch: Optional[int] = None, vocab: Optional[int] = None,
                 top_k: Optional[int] = None, device="cuda"):
        self.w = w
        self.device = device
        self.batch = batch or w.batch
        self.vocab = w.vocab if vocab is None else vocab
        self.dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn,
                           n_pos=w.n_pos, batch=self.batch, block=w.block, win_prefix=w.win_prefix,
                           win_suffix=w.win_suffix, n_clusters=w.n_clusters, top_k=top_k or w.top_k,
                           vocab=self.vocab, dtype=B.BF16 if w.dtype == "bf16" else B.F32,
                           resid_fmt=B.RESID_BY_NAME[w.resid])
        self.params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist,
                               mask_id=max(self.vocab - 1, 0), kmeans_iters=w.kmeans_iters,
                               proxy_support=B.PROXY_ACTIVE if w.proxy_support == "active" else B.PROXY_ALL)
        self.h = B.polestar_create(self.dims, self.params)
        self.ws_bytes = B.polestar_workspace_size(self.h)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.tdt = TDT[w.dtype]
        self.keep = []

    def close(self):
        B.polestar_destroy(self.h)

    def pack(self, which: int, src: torch.Tensor) -> torch.Tensor:
        n = B.polestar_weight_packed_size(self.h, which) // src.element_size()
        dst = torch.empty(n, dtype=src.dtype, device=self.device)
        B.polestar_pack_weight(self.h, which, src.contiguous(), dst)
        return dst

    def zeros(self, *shape, dtype=None):
        return torch.zeros(*shape, dtype=dtype or self.tdt, device=self.device)

    @property
    def win_max(self):
        return self.w.win_prefix + self.w.win_suffix


def packed_layer(dev: Dev, W: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    return {
        "w_qkv": dev.pack(B.W_QKV, torch.cat([W["wq"], W["wk"], W["wv"]], 0)),
        "w_o": dev.pack(B.W_O, W["wo"]),
        "w_gu": dev.pack(B.W_GU, torch.cat([W["wg"], W["wu"]], 0)),
        "w_down": dev.pack(B.W_DOWN, W["wd"]),
    }


def layer_struct(P: Dict[str, torch.Tensor]) -> B.Layer:
    L = B.Layer()
    for name in ("w_qkv", "w_o", "w_gu", "w_down", "k_cache", "v_cache", "win_h", "win_codes", "win_scales",
                 "win_z", "win_m", "proxy_logits"):
        t = P.get(name)
        setattr(L, name, t.data_ptr() if t is not None else None)
    return L


def packet(rows=None, idx=None, count=None) -> B.Packet:
    p = B.Packet()
    p.rows = rows.data_ptr() if rows is not None else None
    p.idx = idx.data_ptr() if idx is not None else None
    p.count = count.data_ptr() if count is not None else None
    return p


def weights(w: synth.Workload, layer: int, device="cuda") -> Dict[str, torch.Tensor]:
    return synth.layer_weights(w, layer, device=device)


def oracle_weights(W: Dict[str, torch.Tensor]) -> Dict[str, np.ndarray]:
    return {k: np64(v) for k, v in W.items()}
