"""Seeded synthetic inputs for the drift-scored sparse KV refresh.

This module only *generates* inputs; it holds none of the method's arithmetic.
Both the HIP path's tests/benchmark and the CPU oracle read their inputs from
here, so the two sides see bit-identical tensors.

Generator (counter based, identical on CPU and GPU):
  * ``hash32`` is the "lowbias32" integer finaliser published by C. Wellons
    (hash-prospector): x ^= x>>16; x *= 0x7feb352d; x ^= x>>15;
    x *= 0x846ca68b; x ^= x>>16, all modulo 2**32.  It is evaluated with
    int64 torch ops whose intermediates never exceed 2**49, so CPU and GPU
    give the same bits.
  * element ``i`` of a tensor with stream seed ``s`` draws
    ``h = hash32((hash32(i) + s) mod 2**32)``; its top 16 bits index a table of
    the 65536 standard-normal quantiles Phi^-1((u + 0.5)/65536) (float32),
    and the value is ``float32(table[u] * float32(std))`` — one correctly
    rounded fp32 multiply — optionally rounded to bf16 by torch (RNE).

The workload recipes (shapes, step counts, unmask schedules) follow the five
synthetic configurations the refresh path is measured and checked on; trained
weights and benchmark prompts are not available, so these stand in for them.
"""
from __future__ import annotations

import math
import statistics
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np
import torch

_M32 = 0xFFFFFFFF


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 tensors holding values in [0, 2**32)."""
    lo = (x & 0xFFFF) * c
    hi = (((x >> 16) * c) & 0xFFFF) << 16
    return (lo + hi) & _M32


def hash32(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 finaliser (Wellons) on int64 tensors with values < 2**32."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def hash32_int(v: int) -> int:
    """Scalar Python version of :func:`hash32` (same bits)."""
    v &= _M32
    v ^= v >> 16
    v = (v * 0x7FEB352D) & _M32
    v ^= v >> 15
    v = (v * 0x846CA68B) & _M32
    v ^= v >> 16
    return v


def stream_seed(*tags: int) -> int:
    """Combine integer tags into one 32-bit stream seed."""
    s = 0x2545F491
    for t in tags:
        s = hash32_int((s + (int(t) & _M32) + 0x9E3779B9) & _M32)
    return s


_TABLES: Dict[str, torch.Tensor] = {}


def _normal_table(device) -> torch.Tensor:
    key = str(device)
    if key not in _TABLES:
        if "cpu" not in _TABLES:
            nd = statistics.NormalDist()
            vals = [nd.inv_cdf((u + 0.5) / 65536.0) for u in range(65536)]
            _TABLES["cpu"] = torch.tensor(vals, dtype=torch.float64).to(torch.float32)
        _TABLES[key] = _TABLES["cpu"].to(device)
    return _TABLES[key]


_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f64": torch.float64}


def normal(shape, std: float, seed: int, device="cpu", dtype="f32", offset: int = 0) -> torch.Tensor:
    """Seeded N(0, std^2) tensor (quantile-table generator, see module doc).

    ``offset`` shifts the element counter: the result equals elements
    [offset, offset + numel) of the flat tensor drawn with the same seed.
    """
    shape = tuple(int(s) for s in shape)
    numel = int(np.prod(shape)) if shape else 1
    assert offset + numel < 2**32
    idx = torch.arange(offset, offset + numel, dtype=torch.int64, device=device)
    h = hash32((hash32(idx) + (seed & _M32)) & _M32)
    u = h >> 16
    vals = _normal_table(device)[u] * torch.tensor(std, dtype=torch.float32, device=device)
    return vals.reshape(shape).to(_DTYPES[dtype] if isinstance(dtype, str) else dtype)


# --------------------------------------------------------------------------
# workload recipes
# --------------------------------------------------------------------------
MAT_IDS = {"wq": 0, "wk": 1, "wv": 2, "wo": 3, "wg": 4, "wu": 5, "wd": 6, "wlm": 7}


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    d: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    prompt: int
    gen: int
    n_layers: int            # layers in the stack; single-layer workloads use 1
    dtype: str               # "f32" or "bf16"
    steps: int
    batch: int = 1
    block: int = 32
    win_prefix: int = 64
    win_suffix: int = 32
    n_clusters: int = 8
    top_k: int = 4
    tau_upd: int = 3
    hist: int = 5
    alpha: float = 10.0
    tau_s: float = 0.9
    tau_suf: float = 0.9
    kmeans_iters: int = 10
    resid: str = "raw"        # "raw", "nvfp4", "fp8", "mxint8" or "mxfp4"
    vocab: int = 0
    unmask_pmf: Tuple[float, ...] = (1.0, 1.0, 1.0, 1.0)   # over counts 1..len
    noise_var: float = 0.1
    single_layer_next: bool = False   # also instantiate layer l+1 (norm, W_K, W_V, KV, window)
    rms_eps: float = 1e-6
    proxy_support: str = "all"        # keys of the proxy attention: "all" positions or the "active" block

    @property
    def n_pos(self) -> int:
        return self.prompt + self.gen

    @property
    def weight_std(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def seed(self, run: int = 0) -> int:
        return 20261202 + 1000 * self.cfg_id + run


WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_fp32_layer", 1, d=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=768,
                prompt=64, gen=256, n_layers=1, dtype="f32", steps=16, single_layer_next=True),
    2: Workload("llada8b_layer", 2, d=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn=12288,
                prompt=512, gen=256, n_layers=1, dtype="bf16", steps=32, single_layer_next=True),
    3: Workload("llada8b_stack32", 3, d=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn=12288,
                prompt=512, gen=512, n_layers=32, dtype="bf16", steps=64,
                unmask_pmf=(1.0, 2.0, 4.0, 2.0, 1.0, 1.0)),
    4: Workload("dream7b_gqa_stack28", 4, d=3584, n_heads=28, n_kv_heads=4, head_dim=128, ffn=18944,
                prompt=384, gen=256, n_layers=28, dtype="bf16", steps=48),
    5: Workload("llada8b_batch16_nvfp4_commit", 5, d=4096, n_heads=32, n_kv_heads=32, head_dim=128,
                ffn=12288, prompt=512, gen=256, n_layers=32, dtype="bf16", steps=32, batch=16,
                resid="nvfp4", vocab=126464),
}


def shrink(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return replace(w, **kw)


def weight(w: Workload, layer: int, mat: str, run: int = 0, device="cpu", dtype=None) -> torch.Tensor:
    """Layer weight in [out, in] (nn.Linear) layout, N(0, 1/d) per element."""
    d, hq, hkv, dh, f = w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn
    shapes = {"wq": (hq * dh, d), "wk": (hkv * dh, d), "wv": (hkv * dh, d), "wo": (d, hq * dh),
              "wg": (f, d), "wu": (f, d), "wd": (d, f), "wlm": (w.vocab, d)}
    seed = stream_seed(w.seed(run), 1, layer, MAT_IDS[mat])
    return normal(shapes[mat], w.weight_std, seed, device, dtype or w.dtype)


def weight_rows(w: Workload, layer: int, mat: str, r0: int, r1: int, run: int = 0, device="cpu",
                dtype=None) -> torch.Tensor:
    """Rows [r0, r1) of :func:`weight` without drawing the whole matrix."""
    cols = {"wq": w.d, "wk": w.d, "wv": w.d, "wo": w.n_heads * w.head_dim, "wg": w.d, "wu": w.d, "wd": w.ffn,
            "wlm": w.d}[mat]
    seed = stream_seed(w.seed(run), 1, layer, MAT_IDS[mat])
    return normal((r1 - r0, cols), w.weight_std, seed, device, dtype or w.dtype, offset=r0 * cols)


def layer_weights(w: Workload, layer: int, run: int = 0, device="cpu", dtype=None) -> Dict[str, torch.Tensor]:
    return {m: weight(w, layer, m, run, device, dtype) for m in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}


def embeddings(w: Workload, run: int = 0, device="cpu", seq: int = 0) -> torch.Tensor:
    """Layer-0 input hidden states for all positions, N(0, 1) (fp32)."""
    return normal((w.n_pos, w.d), 1.0, stream_seed(w.seed(run), 2, seq), device, "f32")


def tensor(w: Workload, tag: Tuple[int, ...], shape, std=1.0, run: int = 0, device="cpu", dtype="f32"):
    """Generic seeded N(0, std^2) tensor for a named synthetic state piece."""
    return normal(shape, std, stream_seed(w.seed(run), 3, *tag), device, dtype)


def unmask_noise(w: Workload, step: int, pos: int, run: int = 0, seq: int = 0, device="cpu") -> torch.Tensor:
    """Perturbation added to a position's input when it is unmasked: N(0, noise_var)."""
    return normal((w.d,), math.sqrt(w.noise_var), stream_seed(w.seed(run), 4, seq, step, pos), device, "f32")


def host_rng(w: Workload, run: int = 0, stream: int = 0) -> np.random.Generator:
    """Host-side seeded generator for discrete choices (unmask schedule, k-means init)."""
    return np.random.default_rng([w.seed(run), stream])


def unmask_schedule(w: Workload, run: int = 0, steps: Optional[int] = None):
    """Per-step list of J_b offsets to unmask, drawn until every block is decoded.

    Counts come from ``w.unmask_pmf`` over {1..len(pmf)}; positions are uniform
    over the still-masked offsets of the active block.  Returns a list of
    (block_index, [offsets]) with one entry per denoising step.
    """
    rng = host_rng(w, run, 1)
    pmf = np.asarray(w.unmask_pmf, dtype=np.float64)
    pmf = pmf / pmf.sum()
    n_blocks = w.gen // w.block
    out = []
    b = 0
    masked = list(range(w.block))
    total = steps if steps is not None else w.steps
    while len(out) < total and b < n_blocks:
        cnt = int(rng.choice(len(pmf), p=pmf)) + 1
        cnt = min(cnt, len(masked))
        pick = sorted(rng.choice(masked, size=cnt, replace=False).tolist())
        out.append((b, pick))
        masked = [m for m in masked if m not in pick]
        if not masked:
            b += 1
            masked = list(range(w.block))
    return out


def kmeans_init(w: Workload, n_win: int, layer: int, block: int, run: int = 0, seq: int = 0) -> np.ndarray:
    """Seeded choice of min(K, n_win) distinct initial centroid rows."""
    rng = np.random.default_rng([w.seed(run), 5, layer, block, seq])
    k_eff = min(w.n_clusters, n_win)
    return rng.permutation(n_win)[:k_eff].astype(np.int32)
