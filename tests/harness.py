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
# isolated near-midpoints move downstream elements by a few such ulps; rows as a
# whole stay within the 2e-3 bound.
BF16_ELEM_BOUND = 4 * 2.0 ** -8


def assert_close(a, b, name, rtol=2e-3, dtype="f32"):
    """Rows within rtol normwise; elements within rtol (float32) or a few bf16 ulps (bf16)."""
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
    """Stored tensors: the same bounds; also report how many values differ at all."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    frac = float(np.mean(a != b)) if a.size else 0.0
    log(f"    {name}: {frac:.3%} stored values differ from the oracle's")
    assert_close(a, b, name, rtol, dtype)
    return frac


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


def check_topk(tg, Dg, D_or, topk_or, k, k_eff, tag):
    """Top-k comparison.  The GPU's clusters must follow the rule on its own drift
    values; the selected set must equal the oracle's unless the oracle's margin
    between the k-th selected and the best unselected drift is below 1e-3
    (returns False: both sets are admissible); within the set, the order may
    differ only between drifts equal to 1e-3 relative."""
    kk = min(k, k_eff)
    tg = np.asarray(tg)[:kk]
    assert np.array_equal(tg, O.topk_clusters(Dg, k, k_eff)[:kk]), f"{tag}: top-k does not follow the rule"
    if set(tg.tolist()) != set(np.asarray(topk_or)[:kk].tolist()):
        mg = topk_margin(D_or, topk_or, k_eff)
        if mg < 1e-3:
            log(f"    {tag}: top-k near-tie (oracle margin {mg:.2e})")
            return False
        raise AssertionError(f"{tag}: top-k {tg.tolist()} != oracle {list(topk_or)} (margin {mg:.2e})")
    D_or = np.asarray(D_or, dtype=np.float64)
    for a, b in zip(tg[:-1], tg[1:]):
        assert D_or[a] >= D_or[b] * (1 - 1e-3) - 1e-12, f"{tag}: top-k order {tg.tolist()} vs oracle drift"
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
                               mask_id=max(self.vocab - 1, 0), kmeans_iters=w.kmeans_iters)
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
