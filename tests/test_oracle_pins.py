"""Pins of the CPU oracle against what the page and the mathematics fix.

Each test checks the oracle against something other than itself: a library
routine implemented independently (torch.nn.functional), a closed form, an
exhaustive table built from the format definition, brute force on tiny
inputs, or an identity of the method (k = K equals a dense recompute).
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import polestar_oracle as O

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- KL drift
def test_kl_nonnegative_and_zero_on_identical():
    for _ in range(50):
        n = int(RNG.integers(2, 64))
        s = RNG.normal(size=(3, n)) * RNG.uniform(0.1, 5)
        sp = RNG.normal(size=(3, n)) * RNG.uniform(0.1, 5)
        kl = O.kl_logits(s, sp)
        assert np.all(kl >= -1e-12)
        assert np.all(O.kl_logits(s, s) == 0.0)


def test_kl_two_key_closed_form():
    # KL between Bernoulli(p) and Bernoulli(q) written from scratch.
    for a, b, a2, b2 in RNG.normal(size=(40, 4)) * 2:
        p = 1.0 / (1.0 + math.exp(-(a - b)))
        q = 1.0 / (1.0 + math.exp(-(a2 - b2)))
        want = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
        got = O.kl_logits(np.array([a, b]), np.array([a2, b2]))
        assert abs(got - want) <= 1e-12 * max(1.0, abs(want))


def test_kl_pinsker_and_shift_invariance():
    for _ in range(50):
        n = int(RNG.integers(2, 200))
        s = RNG.normal(size=n) * 2
        sp = s + RNG.normal(size=n) * RNG.uniform(0.01, 2)
        kl = float(O.kl_logits(s, sp))
        p = np.exp(s - s.max()); p /= p.sum()
        q = np.exp(sp - sp.max()); q /= q.sum()
        assert np.abs(p - q).sum() <= math.sqrt(2 * kl) + 1e-12          # Prop. 2 (Pinsker)
        c1, c2 = RNG.normal(size=2) * 10
        assert abs(float(O.kl_logits(s + c1, sp + c2)) - kl) <= 1e-10 * max(1, kl)


def test_head_summed_drift_clamps_and_sums():
    s = RNG.normal(size=(4, 3, 17))
    sp = RNG.normal(size=(4, 3, 17))
    kl = O.kl_logits(s, sp)
    assert np.allclose(O.head_summed_drift(s, sp), kl.sum(axis=1))


# ---------------------------------------------------------------- layer pieces vs torch
def test_rmsnorm_and_project_match_torch():
    x = RNG.normal(size=(7, 48))
    w = RNG.normal(size=(20, 48))
    eps = 1e-6
    tx = torch.tensor(x)
    want_n = F.rms_norm(tx, (48,), eps=eps).numpy()
    assert np.allclose(O.rmsnorm(x, eps), want_n, rtol=1e-13, atol=0)
    want_p = F.linear(F.rms_norm(tx, (48,), eps=eps), torch.tensor(w)).numpy()
    assert np.allclose(O.project(x, w, eps), want_p, rtol=1e-12, atol=1e-13)


def test_silu_matches_torch():
    x = RNG.normal(size=100) * 5
    assert np.allclose(O.silu(x), F.silu(torch.tensor(x)).numpy(), rtol=1e-14, atol=0)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (28, 4)])
def test_attention_matches_torch_sdpa(hq, hkv):
    n, dh, R = 19, 16, 5
    q = RNG.normal(size=(R, hq, dh))
    k = RNG.normal(size=(n, hkv, dh))
    v = RNG.normal(size=(n, hkv, dh))
    out, logits = O.attention(q, k, v, hq, hkv)
    tq = torch.tensor(q).permute(1, 0, 2)                       # [H, R, dh]
    rep = hq // hkv
    tk = torch.tensor(k).permute(1, 0, 2).repeat_interleave(rep, dim=0)
    tv = torch.tensor(v).permute(1, 0, 2).repeat_interleave(rep, dim=0)
    want = F.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)
    assert np.allclose(logits, np.einsum("rhd,hnd->rhn", q, tk.numpy()) / math.sqrt(dh))


def test_attention_single_key_and_permutations():
    q = RNG.normal(size=(3, 2, 8))
    k = RNG.normal(size=(1, 2, 8))
    v = RNG.normal(size=(1, 2, 8))
    out, _ = O.attention(q, k, v, 2, 2)
    assert np.allclose(out, np.broadcast_to(v[0], out.shape))
    k = RNG.normal(size=(9, 2, 8)); v = RNG.normal(size=(9, 2, 8))
    out, _ = O.attention(q, k, v, 2, 2)
    perm = RNG.permutation(9)
    out2, _ = O.attention(q, k[perm], v[perm], 2, 2)
    assert np.allclose(out, out2)
    qp = RNG.permutation(3)
    out3, _ = O.attention(q[qp], k, v, 2, 2)
    assert np.allclose(out3, out[qp])


def test_full_forward_one_layer_matches_torch_modules():
    d, hq, hkv, dh, f, n = 32, 4, 2, 8, 48, 11
    cfg = O.Cfg(d=d, n_heads=hq, n_kv_heads=hkv, head_dim=dh, ffn=f, n_pos=n, block=4,
                win_prefix=4, win_suffix=2, n_clusters=2, top_k=1, dtype="f64")
    W = {"wq": RNG.normal(size=(hq * dh, d)) / 6, "wk": RNG.normal(size=(hkv * dh, d)) / 6,
         "wv": RNG.normal(size=(hkv * dh, d)) / 6, "wo": RNG.normal(size=(d, hq * dh)) / 6,
         "wg": RNG.normal(size=(f, d)) / 6, "wu": RNG.normal(size=(f, d)) / 6, "wd": RNG.normal(size=(d, f)) / 6}
    h0 = RNG.normal(size=(n, d))
    Hs, Ks, Vs, _ = O.full_forward(h0, [W], cfg)
    T = {k: torch.tensor(v) for k, v in W.items()}
    x = torch.tensor(h0)
    a = F.rms_norm(x, (d,), eps=1e-6)
    q = F.linear(a, T["wq"]).view(n, hq, dh).permute(1, 0, 2)
    k = F.linear(a, T["wk"]).view(n, hkv, dh).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    v = F.linear(a, T["wv"]).view(n, hkv, dh).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    o = F.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).reshape(n, hq * dh)
    hp = x + F.linear(o, T["wo"])
    b = F.rms_norm(hp, (d,), eps=1e-6)
    out = hp + F.linear(F.silu(F.linear(b, T["wg"])) * F.linear(b, T["wu"]), T["wd"])
    assert np.allclose(Hs[1], out.numpy(), rtol=1e-11, atol=1e-11)


# The bf16 storage points of a layer: the rounded RMSNorm output of the stored input row as
# the input of the Q/K/V projections, K and V (the cache) and the layer output.  Queries, the
# attention output, h', RMSNorm(h') and the SwiGLU product stay unrounded.
BF16_POINTS = ("a", "k", "v", "out")


def _torch_layer_bf16(x, T, hq, hkv, dh, skip=None):
    """One layer in float64 torch modules with a bfloat16 cast at each named point."""
    def c(t, name):
        return t if name == skip else t.to(torch.bfloat16).to(torch.float64)
    n, d = x.shape
    a = c(F.rms_norm(x, (d,), eps=1e-6), "a")
    q = F.linear(a, T["wq"]).view(n, hq, dh).permute(1, 0, 2)
    k = c(F.linear(a, T["wk"]), "k").view(n, hkv, dh).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    v = c(F.linear(a, T["wv"]), "v").view(n, hkv, dh).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    o = F.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).reshape(n, hq * dh)
    hp = x + F.linear(o, T["wo"])
    b = F.rms_norm(hp, (d,), eps=1e-6)
    act = F.silu(F.linear(b, T["wg"])) * F.linear(b, T["wu"])
    return c(hp + F.linear(act, T["wd"]), "out")


def test_full_forward_bf16_rounds_at_the_storage_points():
    d, hq, hkv, dh, f, n = 32, 4, 2, 8, 48, 11
    cfg = O.Cfg(d=d, n_heads=hq, n_kv_heads=hkv, head_dim=dh, ffn=f, n_pos=n, block=4,
                win_prefix=4, win_suffix=2, n_clusters=2, top_k=1, dtype="bf16")
    rng = np.random.default_rng(41)
    W = {"wq": rng.normal(size=(hq * dh, d)) / 6, "wk": rng.normal(size=(hkv * dh, d)) / 6,
         "wv": rng.normal(size=(hkv * dh, d)) / 6, "wo": rng.normal(size=(d, hq * dh)) / 6,
         "wg": rng.normal(size=(f, d)) / 6, "wu": rng.normal(size=(f, d)) / 6, "wd": rng.normal(size=(d, f)) / 6}
    h0 = O.round_bf16(rng.normal(size=(n, d)))
    Hs, Ks, Vs, _ = O.full_forward(h0, [W], cfg)
    T = {k: torch.tensor(v) for k, v in W.items()}
    want = _torch_layer_bf16(torch.tensor(h0), T, hq, hkv, dh).numpy()
    assert np.array_equal(O.round_bf16(Hs[1]), Hs[1])
    assert np.allclose(Hs[1], want, rtol=1e-12, atol=1e-12)
    # every point matters: dropping any one cast moves the output off the oracle's
    for p in BF16_POINTS:
        other = _torch_layer_bf16(torch.tensor(h0), T, hq, hkv, dh, skip=p).numpy()
        assert not np.allclose(Hs[1], other, rtol=0, atol=1e-9), f"rounding of {p} has no effect"


# ---------------------------------------------------------------- block-entry forward
def test_entry_positions_cover_window_and_block():
    n, B, pre, suf = 40, 4, 8, 4
    assert np.array_equal(O.entry_positions(12, n, B, pre, suf, True), np.arange(n))
    assert np.array_equal(O.entry_positions(12, n, B, pre, suf, False), np.arange(4, 20))
    assert np.array_equal(O.entry_positions(0, n, B, pre, suf, False), np.arange(0, 8))      # prefix cut at 0
    assert np.array_equal(O.entry_positions(36, n, B, pre, suf, False), np.arange(28, 40))   # suffix cut at n
    for blk in range(0, n - B + 1, B):
        both = np.sort(np.concatenate([O.window_positions(blk, n, B, pre, suf), O.active_positions(blk, B)]))
        assert np.array_equal(O.entry_positions(blk, n, B, pre, suf, False), both)


def _torch_rows_bf16(x_rows, pos, k_all, v_all, T, hq, hkv, dh):
    """Layer rows at positions pos in float64 torch modules, bf16 casts at the storage points;
    k_all/v_all [n, Hkv*dh] hold the other positions' keys and values."""
    c = lambda t: t.to(torch.bfloat16).to(torch.float64)
    r, d = x_rows.shape
    a = c(F.rms_norm(x_rows, (d,), eps=1e-6))
    k_all, v_all = k_all.clone(), v_all.clone()
    k_all[pos] = c(F.linear(a, T["wk"]))
    v_all[pos] = c(F.linear(a, T["wv"]))
    n = k_all.shape[0]
    q = F.linear(a, T["wq"]).view(r, hq, dh).permute(1, 0, 2)
    k = k_all.view(n, hkv, dh).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    v = v_all.view(n, hkv, dh).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
    o = F.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).reshape(r, hq * dh)
    hp = x_rows + F.linear(o, T["wo"])
    b = F.rms_norm(hp, (d,), eps=1e-6)
    act = F.silu(F.linear(b, T["wg"])) * F.linear(b, T["wu"])
    return c(hp + F.linear(act, T["wd"])), k_all, v_all


@pytest.mark.parametrize("full", [True, False])
def test_layer_forward_rows_matches_torch_modules(full):
    # Rows of the entry set against torch modules; the other cache positions hold stale keys and
    # values that the rows must attend to and leave untouched.
    d, hq, hkv, dh, f, n, B, pre, suf = 32, 4, 2, 8, 48, 23, 4, 8, 4
    cfg = O.Cfg(d=d, n_heads=hq, n_kv_heads=hkv, head_dim=dh, ffn=f, n_pos=n, block=B,
                win_prefix=pre, win_suffix=suf, n_clusters=2, top_k=1, dtype="bf16")
    rng = np.random.default_rng(57)
    W = {"wq": rng.normal(size=(hq * dh, d)) / 6, "wk": rng.normal(size=(hkv * dh, d)) / 6,
         "wv": rng.normal(size=(hkv * dh, d)) / 6, "wo": rng.normal(size=(d, hq * dh)) / 6,
         "wg": rng.normal(size=(f, d)) / 6, "wu": rng.normal(size=(f, d)) / 6, "wd": rng.normal(size=(d, f)) / 6}
    h = O.round_bf16(rng.normal(size=(n, d)))
    k_old = O.round_bf16(rng.normal(size=(n, hkv, dh)))
    v_old = O.round_bf16(rng.normal(size=(n, hkv, dh)))
    pos = O.entry_positions(8, n, B, pre, suf, full)
    K, V = k_old.copy(), v_old.copy()
    got = O.layer_forward_rows(h[pos], pos, W, cfg, K, V)
    T = {k: torch.tensor(v) for k, v in W.items()}
    want, kw, vw = _torch_rows_bf16(torch.tensor(h[pos]), torch.tensor(pos), torch.tensor(k_old.reshape(n, -1)),
                                    torch.tensor(v_old.reshape(n, -1)), T, hq, hkv, dh)
    assert np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    assert np.array_equal(K.reshape(n, -1), kw.numpy()) and np.array_equal(V.reshape(n, -1), vw.numpy())
    rest = np.setdiff1d(np.arange(n), pos)
    assert np.array_equal(K[rest], k_old[rest]) and np.array_equal(V[rest], v_old[rest])
    if not full:
        # with the stale rows replaced by the dense forward's, the window rows equal the dense rows
        Hs, Ks, Vs, _ = O.full_forward(h, [W], cfg)
        K2, V2 = Ks[0].copy(), Vs[0].copy()
        K2[pos], V2[pos] = k_old[pos], v_old[pos]
        assert np.allclose(O.layer_forward_rows(h[pos], pos, W, cfg, K2, V2), Hs[1][pos], rtol=0, atol=1e-12)
        assert not np.allclose(got, Hs[1][pos], rtol=0, atol=1e-6)


# ---------------------------------------------------------------- rounding
def test_round_bf16_matches_torch_on_fp32_values():
    x = (RNG.normal(size=20000) * np.exp(RNG.uniform(-20, 20, size=20000))).astype(np.float32)
    want = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_rounds_once_from_float64():
    # 1 + 2^-8 is the exact bf16 midpoint between 1 and 1 + 2^-7: ties to even -> 1.
    assert O.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    # Slightly above the midpoint rounds up even though float32 rounding would land on it.
    v = 1 + 2 ** -8 + 2 ** -40
    assert O.round_bf16(np.array([v]))[0] == 1 + 2 ** -7
    assert O.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6   # tie to even upward


# ---------------------------------------------------------------- spherical k-means
def _objective(x, z, m):
    return float(np.sum(x * z[m]))


def test_kmeans_unit_norm_monotone_and_fixed_point():
    for trial in range(20):
        nw, d, K = int(RNG.integers(9, 60)), int(RNG.integers(3, 40)), int(RNG.integers(2, 9))
        h = RNG.normal(size=(nw, d))
        init = RNG.permutation(nw)[: min(K, nw)]
        z, m, trace = O.spherical_kmeans(h, K, init, iters=10)
        kk = min(K, nw)
        assert np.allclose(np.linalg.norm(z[:kk], axis=1), 1.0, atol=1e-12)
        assert np.all(np.diff(trace) >= -1e-12)
        # objective after an update equals sum of member-sum norms
        x = O.unit_rows(h)
        assert abs(trace[-1] - _objective(x, z, m)) < 1e-9
        # one more assignment from the final centroids at the converged state
        z2, m2, trace2 = O.spherical_kmeans(h, K, init, iters=60)
        cos = x @ z2[:kk].T
        assert np.array_equal(np.argmax(cos, axis=1), m2)


def test_kmeans_recovers_planted_directions():
    d, K, per = 64, 8, 12
    dirs = np.linalg.qr(RNG.normal(size=(d, K)))[0].T          # orthonormal directions
    labels = np.repeat(np.arange(K), per)
    h = dirs[labels] * RNG.uniform(0.5, 3.0, size=(K * per, 1)) + 0.02 * RNG.normal(size=(K * per, d))
    init = np.array([c * per for c in range(K)])
    z, m, _ = O.spherical_kmeans(h, K, init, iters=10)
    assert np.array_equal(m, labels)
    assert np.all(np.sum(z * dirs, axis=1) > 0.99)


def test_kmeans_bruteforce_tiny():
    for trial in range(10):
        nw = int(RNG.integers(4, 10))
        h = RNG.normal(size=(nw, 3))
        x = O.unit_rows(h)
        best = -1.0
        for lab in itertools.product(range(2), repeat=nw):
            lab = np.asarray(lab)
            val = sum(np.linalg.norm(x[lab == c].sum(axis=0)) for c in range(2) if (lab == c).any())
            best = max(best, val)
        z, m, trace = O.spherical_kmeans(h, 2, RNG.permutation(nw)[:2], iters=10)
        assert trace[-1] <= best + 1e-12


def test_kmeans_zero_row_and_empty_cluster():
    h = np.zeros((5, 4)); h[1] = [1, 0, 0, 0]; h[2] = [0, 1, 0, 0]; h[3] = [1, 0.1, 0, 0]; h[4] = [1, 0.2, 0, 0]
    z, m, _ = O.spherical_kmeans(h, 3, np.array([1, 2, 0]), iters=3)
    assert m[0] == 0                                 # zero row -> lowest index
    # cluster 2 starts at the zero row: it keeps its (zero) centroid when empty
    assert np.all(z[2] == 0)


def test_centroid_update_fixed_labels():
    h = RNG.normal(size=(30, 16))
    m = RNG.integers(0, 4, size=30)
    m[m == 3] = 2                                    # cluster 3 empty
    zold = RNG.normal(size=(4, 16))
    z = O.centroid_update(h * RNG.uniform(0.1, 10, size=(30, 1)), m, zold)
    x = h / np.linalg.norm(h, axis=1, keepdims=True)
    for c in range(3):
        s = x[m == c].sum(axis=0)
        assert np.allclose(z[c], s / np.linalg.norm(s))
    assert np.array_equal(z[3], zold[3])


def test_kmeans_fewer_rows_than_clusters():
    h = RNG.normal(size=(5, 8))
    z, m, _ = O.spherical_kmeans(h, 8, np.array([4, 2, 0, 1, 3]), iters=4)
    assert set(m.tolist()) <= set(range(5)) and np.all(z[5:] == 0)


# ---------------------------------------------------------------- NVFP4
def test_e2m1_table_from_bit_fields():
    for code in range(16):
        s, e, mt = code >> 3, (code >> 1) & 3, code & 1
        mag = mt * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + mt / 2)
        assert O.e2m1_value(code) == (-mag if s else mag)


def test_e4m3_table_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_value(codes)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_e4m3_encode_matches_torch_rne():
    x = np.concatenate([np.abs(RNG.normal(size=20000)) * np.exp(RNG.uniform(-12, 6, size=20000)),
                        O.e4m3_value(np.arange(0x7F)),
                        (O.e4m3_value(np.arange(0x7E)) + O.e4m3_value(np.arange(1, 0x7F))) / 2])
    x = x[x <= 448].astype(np.float32).astype(np.float64)
    want = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), want)
    assert O.e4m3_encode(np.array([1e6]))[0] == 0x7E                    # saturates at 448


def test_e2m1_encode_ties_to_even_and_saturation():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for y, v in ties.items():
        assert O.e2m1_value(O.e2m1_encode(np.array([y])))[0] == v
        assert O.e2m1_value(O.e2m1_encode(np.array([-y])))[0] == -v
    grid = O.E2M1_MAG
    for a, b in zip(grid[:-1], grid[1:]):
        mid = (a + b) / 2
        assert O.e2m1_value(O.e2m1_encode(np.array([np.nextafter(mid, 0)])))[0] == a
        assert O.e2m1_value(O.e2m1_encode(np.array([np.nextafter(mid, 10)])))[0] == b
    assert O.e2m1_value(O.e2m1_encode(np.array([7.9, -100.0]))).tolist() == [6.0, -6.0]
    assert O.e2m1_encode(np.array([-0.0, -0.1]))[0] == 0 and O.e2m1_encode(np.array([-0.1]))[0] == 0


def test_nvfp4_exact_round_trip_on_representable_groups():
    rows, d = 12, 128
    grid = np.concatenate([O.E2M1_MAG, -O.E2M1_MAG[1:]])
    vals = RNG.choice(grid, size=(rows, d))
    vals[:, ::16] = RNG.choice([6.0, -6.0], size=(rows, d // 16))       # every group holds +-6
    sc = RNG.integers(1, 0x7E, size=(rows, d // 16))
    sv = O.e4m3_value(sc)
    r = (vals.reshape(rows, d // 16, 16) * sv[..., None]).reshape(rows, d).astype(np.float32)
    packed, scales = O.nvfp4_quantize(r)
    assert np.array_equal(scales, sc.astype(np.uint8))
    assert np.array_equal(O.nvfp4_dequantize(packed, scales), r)


def test_nvfp4_error_bound_and_zero_group():
    r = (RNG.normal(size=(16, 256)) * np.exp(RNG.uniform(-6, 4, size=(16, 1)))).astype(np.float32)
    r[3, 32:48] = 0.0
    packed, scales = O.nvfp4_quantize(r)
    deq = O.nvfp4_dequantize(packed, scales)
    sv = np.repeat(O.e4m3_value(scales), 16, axis=1)
    y = np.abs(r.astype(np.float64)) / np.where(sv > 0, sv, 1)
    step = np.select([y < 2, y < 4], [0.5, 1.0], 2.0)
    err = np.abs(deq.astype(np.float64) - r)
    ok = (err <= sv * step / 2 + 1e-30) | ((y > 6) & np.isclose(err, np.abs(r) - 6 * sv, rtol=1e-6))
    assert ok.all()
    assert np.all(packed[3, 16:24] == 0) and scales[3, 2] == 0


def test_nvfp4_nibble_order():
    r = np.zeros((1, 16), dtype=np.float32)
    r[0, 0], r[0, 1] = 6.0, 0.5          # amax 6 -> s = 1 exactly
    packed, scales = O.nvfp4_quantize(r)
    assert O.e4m3_value(scales)[0, 0] == 1.0
    assert packed[0, 0] == (0x7 | (0x1 << 4))


def test_fp8_codes_match_the_e4m3fn_encoding():
    # OCP E4M3FN: 1.0 = 0x38, 448 = 0x7E (largest finite), 2^-6 = 0x08 (smallest normal),
    # 2^-9 = 0x01 (smallest subnormal); negative values set bit 7; zero is +0
    x = np.array([[1.0, 448.0, 2.0 ** -6, 2.0 ** -9, -1.0, -448.0, 0.0, -0.0]], dtype=np.float32)
    codes, scales = O.fp8_quantize(x)
    assert codes.tolist() == [[0x38, 0x7E, 0x08, 0x01, 0xB8, 0xFE, 0x00, 0x00]] and scales.shape == (1, 0)
    # every finite code round-trips; beyond 448 saturates; ties go to the even mantissa
    mags = O.e4m3_value(np.arange(0x7F)).astype(np.float32)[None]
    assert np.array_equal(O.fp8_quantize(mags)[0][0], np.arange(0x7F, dtype=np.uint8))
    assert np.array_equal(O.fp8_dequantize(O.fp8_quantize(-mags[:, 1:])[0]), -mags[:, 1:])
    assert O.fp8_quantize(np.array([[1000.0, 1.0625, 1.1875]], dtype=np.float32))[0].tolist() == [[0x7E, 0x38, 0x3A]]


def test_mxint8_hand_blocks():
    r = np.zeros((3, 32), dtype=np.float32)
    r[0, :4] = [1.5, -0.75, 0.5, 2.0 ** -7]           # amax 1.5 -> X = 1; 2^-7 * 64 = 0.5 -> 0 (even)
    r[1, :3] = [-2.0, 1.0, 3 * 2.0 ** -6]             # amax 2 -> X = 2; 3*2^-6 / 2 * 64 = 1.5 -> 2
    r[2, :2] = [127.5 / 64, -1.0]                     # 127.5 rounds to 128 -> clamped to 127
    codes, scales = O.mxint8_quantize(r)
    q = codes.astype(np.int64)
    q = np.where(q >= 128, q - 256, q)
    assert q[0, :4].tolist() == [96, -48, 32, 0] and scales[0, 0] == 127
    assert q[1, :3].tolist() == [-64, 32, 2] and scales[1, 0] == 128
    assert q[2, :2].tolist() == [127, -64] and scales[2, 0] == 127
    z, zs = O.mxint8_quantize(np.zeros((1, 32), dtype=np.float32))
    assert not z.any() and zs[0, 0] == 0                # all-zero block: exponent -127
    assert np.array_equal(O.mxint8_dequantize(codes[:1], scales[:1])[0, :3], np.float32([1.5, -0.75, 0.5]))


def test_mxint8_error_bound():
    rng = np.random.default_rng(57)
    r = (rng.normal(size=(8, 256)) * np.exp(rng.uniform(-8, 6, size=(8, 1)))).astype(np.float32)
    codes, scales = O.mxint8_quantize(r)
    deq = O.mxint8_dequantize(codes, scales).astype(np.float64)
    X = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
    # half a step of X * 2^-6, or one step where the largest value is clamped at 127
    assert np.all(np.abs(deq - r) <= X * 2.0 ** -6 + 1e-300)
    assert np.all((np.abs(deq - r) <= X * 2.0 ** -7) | (np.abs(r) >= X * 127 / 64))


def test_mxfp4_hand_blocks_and_round_trip():
    r = np.zeros((3, 32), dtype=np.float32)
    r[0, :3] = [6.0, 0.5, -1.5]                       # amax 6 -> X = 1, exact
    r[1, :2] = [7.0, -0.25]                           # amax 7 -> X = 1: 7 saturates to 6
    r[2, :2] = [0.75, 0.125]                          # amax 0.75 -> X = 1/8: 6 and 1
    packed, scales = O.mxfp4_quantize(r)
    assert (scales[:, 0].astype(int) - 127).tolist() == [0, 0, -3]
    deq = O.mxfp4_dequantize(packed, scales)
    assert deq[0, :3].tolist() == [6.0, 0.5, -1.5] and deq[1, :2].tolist() == [6.0, -0.0]
    assert deq[2, :2].tolist() == [0.75, 0.125]
    assert packed[0, 0] == (0x7 | (0x1 << 4))           # element 2j in the low nibble
    # representable blocks (values on the E2M1 grid times 2^k, each block holding +-4 or +-6)
    rng = np.random.default_rng(58)
    rows, d = 6, 128
    grid = np.concatenate([O.E2M1_MAG, -O.E2M1_MAG[1:]])
    vals = rng.choice(grid, size=(rows, d))
    vals[:, ::32] = rng.choice([4.0, -6.0], size=(rows, d // 32))
    k = rng.integers(-20, 20, size=(rows, d // 32))
    x = np.ldexp(vals.reshape(rows, d // 32, 32), k[..., None]).reshape(rows, d).astype(np.float32)
    p2, s2 = O.mxfp4_quantize(x)
    assert np.array_equal(O.mxfp4_dequantize(p2, s2), x)


def test_kv_staleness_special_cases_and_brute_force():
    rng = np.random.default_rng(61)
    n, H, dh = 7, 3, 8
    k = rng.normal(size=(n, H, dh))
    v = rng.normal(size=(n, H, dh))
    assert np.allclose(O.kv_staleness(k, v, k, v), 0.0, atol=1e-15)                 # fresh cache
    assert np.allclose(O.kv_staleness(k, v, -k, -v), 2.0)                           # opposite rows
    assert np.allclose(O.kv_staleness(2.5 * k, v, k, 0.1 * v), 0.0, atol=1e-15)      # scale invariant
    kr, vr = rng.normal(size=(n, H, dh)), rng.normal(size=(n, H, dh))
    e = O.kv_staleness(k, v, kr, vr)
    for i in range(n):   # per-head cosines written out, then the App. C.2 combination
        ck = [float(k[i, h] @ kr[i, h]) / math.sqrt(float(k[i, h] @ k[i, h]) * float(kr[i, h] @ kr[i, h]))
              for h in range(H)]
        cv = [float(v[i, h] @ vr[i, h]) / math.sqrt(float(v[i, h] @ v[i, h]) * float(vr[i, h] @ vr[i, h]))
              for h in range(H)]
        assert abs(e[i] - (1 - 0.5 * (sum(ck) / H + sum(cv) / H))) < 1e-12
    z = np.zeros((1, H, dh))
    assert np.allclose(O.kv_staleness(z, z, k[:1], v[:1]), 1.0)                      # zero rows: cos 0


def test_selection_accuracy_counts_the_true_top_quarter():
    stale = np.array([0.1, 0.9, 0.3, 0.9, 0.0, 0.5, 0.2, 0.8])
    assert O.top_fraction(stale, 0.25).tolist() == [1, 3]                            # ties -> lower index
    assert O.selection_accuracy([1, 3], stale) == 1.0
    assert O.selection_accuracy([1, 5], stale) == 0.5
    assert O.selection_accuracy([0, 2, 4], stale) == 0.0
    assert O.top_fraction(np.zeros(5), 0.25).tolist() == [0, 1]                      # ceil(1.25) = 2


# ---------------------------------------------------------------- selection
def test_topk_bruteforce_and_ties():
    for _ in range(200):
        K = int(RNG.integers(1, 17))
        k = int(RNG.integers(1, K + 1))
        D = RNG.integers(0, 4, size=K).astype(np.float64)      # many exact ties
        want = np.lexsort((np.arange(K), -D))[:k]
        assert np.array_equal(O.topk_clusters(D, k), want)
    D = RNG.normal(size=8)
    assert sorted(O.topk_clusters(D, 8).tolist()) == list(range(8))
    assert O.topk_clusters(np.zeros(8), 4).tolist() == [0, 1, 2, 3]
    assert O.topk_clusters(np.array([5, 1, 9, 9.0]), 3, k_eff=3).tolist() == [2, 0, 1]


def test_select_rows_bruteforce():
    m = RNG.integers(0, 8, size=96)
    top = np.array([6, 1, 3, 0])
    want = np.nonzero(np.isin(m, top))[0]
    assert np.array_equal(O.select_rows(m, top), want)


def test_window_positions_bruteforce():
    for n, s, B, pre, suf in [(320, 64, 32, 64, 32), (100, 0, 32, 64, 32), (96, 64, 32, 64, 32),
                              (1024, 992, 32, 64, 32), (50, 30, 8, 16, 8)]:
        want = [j for j in range(n) if s - pre <= j < s + B + suf and not (s <= j < s + B)]
        assert O.window_positions(s, n, B, pre, suf).tolist() == want


def test_trigger_truth_table():
    assert [O.should_refresh(c, 3) for c in range(7)] == [False] * 4 + [True] * 3
    assert not O.should_refresh(10**6, None)
    assert O.should_refresh(1, 0) and not O.should_refresh(0, 0)


# ---------------------------------------------------------------- commit
def test_commit_threshold_limits_and_boundaries():
    f = np.float32
    tau_s, alpha = 0.9, 10.0
    # tau_d = 0 at c = tau_s, and alpha * tau_s^2 at c = 0
    _, _, taud, _, _ = O.commit_decide([0.0, 0.0], [f(tau_s), 0.0], [1, 1], np.zeros((2, 5)), [0, 0], 5, alpha, tau_s)
    assert taud[0] == 0.0 and abs(taud[1] - alpha * tau_s ** 2) < 1e-5
    # c exactly tau_s commits (c >= tau_s); spike exactly tau_d does not (strict >)
    c = np.array([f(tau_s), f(0.5), f(0.5), f(0.95)])
    td = f(f(alpha) * f(f(f(tau_s) - f(0.5)) ** 2))
    delta = np.array([0.0, td, np.nextafter(td, np.float32(10)), 0.0], dtype=np.float32)
    commit, spike, _, _, _ = O.commit_decide(delta, c, [1, 1, 1, 0], np.zeros((4, 5)), [0] * 4, 5, alpha, tau_s)
    assert commit.tolist() == [1, 0, 1, 0]            # last one is not masked


def test_commit_history_mean_and_ring():
    hv = np.zeros((1, 3), dtype=np.float32)
    hc = np.zeros(1, dtype=np.int32)
    seq = [1.0, 2.0, 4.0, 8.0, 16.0]
    spikes = []
    for d in seq:
        _, sp, _, hv, hc = O.commit_decide([d], [0.0], [1], hv, hc, 3, 10.0, 0.9)
        spikes.append(float(sp[0]))
    # history holds the previous <= 3 deltas; its mean is subtracted
    assert np.allclose(spikes, [1.0, 1.0, 2.5, 8.0 - 7.0 / 3.0, 16.0 - 14.0 / 3.0], rtol=1e-6)
    assert hv[0].tolist() == [4.0, 8.0, 16.0]
    # h = 0: raw drift
    _, sp, _, _, _ = O.commit_decide([3.5], [0.0], [1], np.zeros((1, 1)), [0], 0, 10.0, 0.9)
    assert sp[0] == np.float32(3.5)


def test_confidence_matches_torch_softmax():
    V, d = 50, 16
    x = RNG.normal(size=(6, d))
    w = RNG.normal(size=(V, d))
    x[2] = w[7] * 40                        # planted: id 7 dominates
    c, yhat, _ = O.confidence(x, w, mask_id=V - 1, eps=1e-6)
    p = torch.softmax(F.linear(F.rms_norm(torch.tensor(x), (d,), eps=1e-6), torch.tensor(w)), dim=1).numpy()
    p[:, V - 1] = -1
    assert np.allclose(c, p.max(axis=1), rtol=1e-12)
    assert np.array_equal(yhat, p.argmax(axis=1))
    assert yhat[2] == 7 and c[2] > 0.99
    assert np.all(c >= 1.0 / V - 1e-12) and np.all(c <= 1.0)


def test_suffix_commit_rule():
    out = O.suffix_commit([0.95, 0.9, 0.5, 0.99], [1, 1, 1, 0], 0.9)
    assert out.tolist() == [1, 1, 0, 0]


def test_entry_commit_rule():
    # hand cases: the threshold itself commits, one float32 step below does not, unmasked never
    f = np.float32
    c = [f(0.9), np.nextafter(f(0.9), f(0)), f(0.99), f(0.99)]
    assert O.entry_commit(c, [1, 1, 1, 0], 0.9).tolist() == [1, 0, 1, 0]
    # the in-block rule with no drift and an empty history reduces to it: spike 0 never exceeds
    # tau_d = alpha (tau_s - c)^2 >= 0, so only the confidence can commit
    rng = np.random.default_rng(88)
    for alpha in (2.0, 10.0, 40.0):
        conf = rng.uniform(0.5, 1.0, size=64).astype(np.float32)
        masked = rng.integers(0, 2, size=64)
        com, _, _, _, _ = O.commit_decide(np.zeros(64), conf, masked, np.zeros((64, 5)), np.zeros(64, dtype=int), 5,
                                          alpha, 0.9)
        assert np.array_equal(O.entry_commit(conf, masked, 0.9), com)


# ---------------------------------------------------------------- the k = K identity
def _tiny_stack(n_layers, d=32, hq=4, hkv=2, dh=8, f=48, seed=7):
    rng = np.random.default_rng(seed)
    s = 1 / math.sqrt(d)
    return [{"wq": rng.normal(size=(hq * dh, d)) * s, "wk": rng.normal(size=(hkv * dh, d)) * s,
             "wv": rng.normal(size=(hkv * dh, d)) * s, "wo": rng.normal(size=(d, hq * dh)) * s,
             "wg": rng.normal(size=(f, d)) * s, "wu": rng.normal(size=(f, d)) * s,
             "wd": rng.normal(size=(d, f)) * s} for _ in range(n_layers)]


def _run_refresh_steps(cfg, layers, h0, blk_start, steps, tau_upd, rng, k_override=None):
    """Oracle refresh loop over a stack; returns final per-layer states and h0."""
    n_layers = len(layers)
    Hs, Ks, Vs, _ = O.full_forward(h0, layers, cfg)
    wpos = O.window_positions(blk_start, cfg.n, cfg.B, cfg.pre, cfg.suf)
    states = []
    for l in range(n_layers):
        init = rng.permutation(len(wpos))[: min(cfg.K, len(wpos))]
        states.append(O.block_entry_layer_state(Hs[l], Ks[l], Vs[l], layers[l]["wq"], cfg, blk_start, init))
    h0 = h0.copy()
    decoded = 0
    for t in range(steps):
        pos = blk_start + rng.choice(cfg.B, size=2, replace=False)
        h0[pos] += rng.normal(size=(2, cfg.d)) * 0.3
        decoded += 2
        refresh = O.should_refresh(decoded, tau_upd)
        if refresh:
            decoded = 0
        h_act = cfg.st(h0[blk_start: blk_start + cfg.B])
        u_rows, u_idx = None, None
        for l in range(n_layers):
            ls = states[l]
            if refresh:
                cu = O.cluster_update(ls, cfg, u_rows, u_idx)
                dr = O.drift_layer(ls, layers[l], cfg, blk_start, h_act, cu["h"], cu["patched"], True)
                S = dr["S"]
                rf = O.refresh_layer(layers[l], cfg, h_act, cu["h"], dr["o"], S)
                u_rows, u_idx = rf["U"], S
            else:
                dr = O.drift_layer(ls, layers[l], cfg, blk_start, h_act, None, None, False)
                rf = O.refresh_layer(layers[l], cfg, h_act, np.zeros((0, cfg.d)), dr["o"], np.zeros(0, int))
            h_act = rf["h_act_out"]
    return states, h0, h_act


def test_refresh_with_k_equal_K_matches_dense_recompute():
    # prompt 64 + gen 64, B = 32, block 0: the window covers every non-active position.
    layers = _tiny_stack(3)
    cfg = O.Cfg(d=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48, n_pos=128, block=32, win_prefix=64,
                win_suffix=32, n_clusters=8, top_k=8, dtype="f64")
    rng = np.random.default_rng(3)
    h0 = rng.normal(size=(128, 32))
    states, h0_final, h_act = _run_refresh_steps(cfg, layers, h0, 64, steps=4, tau_upd=0, rng=rng)
    Hs, Ks, Vs, _ = O.full_forward(h0_final, layers, cfg)
    wpos = O.window_positions(64, 128, 32, 64, 32)
    for l in range(3):
        assert np.allclose(states[l]["K"], Ks[l], rtol=0, atol=1e-11)
        assert np.allclose(states[l]["V"], Vs[l], rtol=0, atol=1e-11)
        assert np.allclose(states[l]["H"], Hs[l][wpos], rtol=0, atol=1e-11)
    assert np.allclose(h_act, Hs[3][64:96], atol=1e-11)


def test_refresh_with_k_below_K_is_not_dense():
    # sanity: the identity above is not vacuous; k < K leaves stale rows behind.
    layers = _tiny_stack(3)
    cfg = O.Cfg(d=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48, n_pos=128, block=32, win_prefix=64,
                win_suffix=32, n_clusters=8, top_k=2, dtype="f64")
    rng = np.random.default_rng(3)
    h0 = rng.normal(size=(128, 32))
    states, h0_final, _ = _run_refresh_steps(cfg, layers, h0, 64, steps=4, tau_upd=0, rng=rng)
    Hs, Ks, _, _ = O.full_forward(h0_final, layers, cfg)
    assert not np.allclose(states[2]["K"], Ks[2], atol=1e-6)


def test_no_refresh_leaves_window_caches_untouched():
    layers = _tiny_stack(2)
    cfg = O.Cfg(d=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48, n_pos=128, block=32, win_prefix=64,
                win_suffix=32, n_clusters=8, top_k=4, dtype="bf16")
    rng = np.random.default_rng(5)
    h0 = rng.normal(size=(128, 32))
    Hs, Ks, Vs, _ = O.full_forward(h0, layers, cfg)
    rng2 = np.random.default_rng(5)
    rng2.normal(size=(128, 32))
    states, _, _ = _run_refresh_steps(cfg, layers, h0, 64, steps=3, tau_upd=None, rng=rng2)
    jb = np.arange(64, 96)
    other = np.setdiff1d(np.arange(128), jb)
    for l in range(2):
        assert np.array_equal(states[l]["K"][other], Ks[l][other])
        assert np.array_equal(states[l]["V"][other], Vs[l][other])
        assert np.array_equal(states[l]["H"], Hs[l][O.window_positions(64, 128, 32, 64, 32)])


def test_kv_rows_follow_fresh_packet():
    cfg = O.Cfg(d=32, n_heads=4, n_kv_heads=2, head_dim=8, ffn=48, n_pos=128, block=32, win_prefix=64,
                win_suffix=32, n_clusters=8, top_k=4, dtype="bf16")
    u = O.round_bf16(RNG.normal(size=(5, 32)))
    wk, wv = RNG.normal(size=(16, 32)), RNG.normal(size=(16, 32))
    k, v = O.kv_rows(u, wk, wv, cfg)
    a = F.rms_norm(torch.tensor(u), (32,), eps=1e-6).to(torch.bfloat16).to(torch.float64)
    want = F.linear(a, torch.tensor(wk)).numpy()
    # the projection of the bf16-rounded normalised rows, itself rounded once to bf16
    assert np.array_equal(O.round_bf16(k.reshape(5, 16)), k.reshape(5, 16))
    assert np.array_equal(k.reshape(5, 16), O.round_bf16(want))


# ---------------------------------------------------------------- pins of the compositions
def test_head_summed_drift_clamps_rounding_negatives():
    """Each head's KL is clamped at 0 before the head sum [Eq. 4 reading: D = sum_h max(0, KL)].

    fp64 rounding makes KL of two nearly equal logit vectors slightly negative about half the
    time; a seeded search finds such a pair, so an unclamped sum would come out negative."""
    rng = np.random.default_rng(7)
    neg = None
    for _ in range(200):
        s = rng.normal(size=40) * 3
        sp = s + rng.normal(size=40) * 1e-9
        if float(O.kl_logits(s, sp)) < 0:
            neg = (s, sp)
            break
    assert neg is not None
    s_same = rng.normal(size=40)
    s_far, sp_far = rng.normal(size=40), rng.normal(size=40)
    kl_far = float(O.kl_logits(s_far, sp_far))
    assert kl_far > 0.1
    heads = np.stack([s_same, neg[0], s_far])[None]          # [1 row, 3 heads, 40 keys]
    heads_prev = np.stack([s_same, neg[1], sp_far])[None]
    kl = O.kl_logits(heads, heads_prev)[0]
    assert kl[0] == 0.0 and kl[1] < 0.0
    # clamped: the negative head adds nothing; without the clamp the first sum would be < 0
    assert O.head_summed_drift(heads[:, :2], heads_prev[:, :2])[0] == 0.0
    assert O.head_summed_drift(heads, heads_prev)[0] == kl_far


def _tiny_layer(dtype="f64", K=2, k=1):
    cfg = O.Cfg(d=32, n_heads=2, n_kv_heads=2, head_dim=16, ffn=48, n_pos=20, block=4, win_prefix=8,
                win_suffix=4, n_clusters=K, top_k=k, dtype=dtype)
    rng = np.random.default_rng(11)
    W = {"wq": rng.normal(size=(32, 32)) / 6, "wk": rng.normal(size=(32, 32)) / 6,
         "wv": rng.normal(size=(32, 32)) / 6, "wo": rng.normal(size=(32, 32)) / 6,
         "wg": rng.normal(size=(48, 32)) / 6, "wu": rng.normal(size=(48, 32)) / 6,
         "wd": rng.normal(size=(32, 48)) / 7}
    blk = 8
    nw = len(O.window_positions(blk, cfg.n, cfg.B, cfg.pre, cfg.suf))
    H = rng.normal(size=(nw, 32))
    z, m, _ = O.spherical_kmeans(H, K, np.arange(K), 10)
    ls = {"K": rng.normal(size=(20, 2, 16)), "V": rng.normal(size=(20, 2, 16)),
          "P": O.round_f32(rng.normal(size=(K, 2, 20)) * 3), "Z": cfg.st(z), "M": m, "H": H}
    return cfg, W, ls, blk, rng.normal(size=(4, 32)), H


def test_drift_reference_is_replaced_after_the_kl():
    """The drift compares this step's proxy logits with the reference and only then stores them as
    the next reference [Algorithm 1: P_t is measured against P_{t-1}, then kept].

    First call against a random reference: a clearly positive drift.  A second call on the
    unchanged state compares the recomputed logits with their own float32 copy, so its drift is
    zero up to that rounding.  Storing before the KL would make the first drift zero too; not
    storing would repeat the first drift."""
    cfg, W, ls, blk, h_act, H = _tiny_layer()
    no_patch = np.zeros(len(H), dtype=bool)
    r1 = O.drift_layer(ls, W, cfg, blk, h_act, H, no_patch, True)
    assert np.array_equal(ls["P"], O.round_f32(r1["proxy_logits"]))
    assert r1["D"].min() > 0.1
    r2 = O.drift_layer(ls, W, cfg, blk, h_act, H, no_patch, True)
    assert np.array_equal(r2["proxy_logits"], r1["proxy_logits"])
    assert r2["D"].max() <= 1e-9


def _grid_residuals(fmt, rows, d, rng):
    """Residual rows that the format represents exactly, with every block's scale attained."""
    if fmt == "fp8":
        # E4M3 values m/8 * 2^e, e in [-4, -2]: multiples of 2^-7 below 0.5
        mant = rng.integers(8, 16, size=(rows, d)) / 8.0
        r = mant * np.ldexp(1.0, rng.integers(-4, -1, size=(rows, d))) * rng.choice([-1, 1], size=(rows, d))
        r[rng.random(size=(rows, d)) < 0.1] = 0.0
        return r
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    G = 16 if fmt == "nvfp4" else 32
    r = np.zeros((rows, d))
    for i in range(rows):
        for g0 in range(0, d, G):
            if fmt == "mxint8":
                X = 2.0 ** -2                        # amax in [2^-2, 2^-1): q_max in [64, 127]
                q = rng.integers(-63, 64, size=G)
                q[rng.integers(G)] = int(rng.choice([-1, 1]) * rng.integers(64, 128))
                r[i, g0:g0 + G] = q * X / 64
                continue
            if fmt == "nvfp4":
                sc = float(rng.choice([2.0 ** -4, 2.0 ** -3, 1.5 * 2.0 ** -4]))   # E4M3 values
                top = 6.0                            # amax / 6 is the scale itself
            else:                                    # mxfp4: X = 2^(floor(log2 amax) - 2)
                sc = 2.0 ** -4
                top = float(rng.choice([4.0, 6.0]))
            g = rng.choice(grid[grid <= top], size=G) * rng.choice([-1, 1], size=G)
            g[rng.integers(G)] = top * rng.choice([-1, 1])
            r[i, g0:g0 + G] = g * sc
    return r


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8", "mxint8", "mxfp4"])
def test_residual_composition_exact_round_trip(fmt):
    """Window rows stored as residuals to their own cluster's centroid and rebuilt by adding that
    centroid back [§4.1 "Cluster and Quantize Hidden States"; App. C.3]: on residuals the format
    represents exactly, rebuild(quantise(h - z_M(i))) == h bit for bit, and the codes decode to
    h - z_M(i).  Subtracting another cluster's centroid, or rebuilding without the centroid,
    breaks both (checked on the same rows)."""
    rng = np.random.default_rng(5)
    rows, d, K = 9, 64, 3
    z = rng.integers(-8, 9, size=(K, d)) / 16.0          # bf16-exact, distinct per cluster
    m = np.arange(rows) % K
    r = _grid_residuals(fmt, rows, d, rng)
    h = z[m] + r
    assert np.array_equal(O.round_bf16(h), h)              # the rows are bf16 values
    codes, scales = O.residual_quantize(h, z, m, fmt)
    deq = O.RESID_CODECS[fmt][1](codes, scales).astype(np.float64)
    assert np.array_equal(deq, r)
    back = O.residual_dequantize(codes, scales, z, m, O.round_bf16, fmt)
    assert np.array_equal(back, h)
    # the mistakes this pins: the wrong centroid, or none, at either end
    wrong = (m + 1) % K
    c2, s2 = O.residual_quantize(h, z, wrong, fmt)
    assert not np.array_equal(O.residual_dequantize(c2, s2, z, wrong, O.round_bf16, fmt), h)
    assert not np.array_equal(O.residual_dequantize(codes, scales, np.zeros_like(z), m, O.round_bf16, fmt), h)


def test_proxy_drift_over_the_active_block_keys():
    """Proxy attention over the active block's keys only [§4.1 "Measuring Drift..."; Eq. 3, the
    "active" reading of the key support]: the KL equals torch's kl_div between the softmaxes of
    the J_b scores; keys outside J_b do not move D ("active") but do move it ("all")."""
    rng = np.random.default_rng(3)
    n, hq, dh, K, blk, Bk = 40, 2, 16, 3, 12, 8
    common = dict(d=32, n_heads=hq, n_kv_heads=hq, head_dim=dh, ffn=48, n_pos=n, block=Bk, win_prefix=8,
                  win_suffix=4, n_clusters=K, top_k=1, dtype="f64")
    act = O.Cfg(proxy_support="active", **common)
    full = O.Cfg(proxy_support="all", **common)
    zq = rng.normal(size=(K, hq, dh))
    Kc, Vc = rng.normal(size=(n, hq, dh)), rng.normal(size=(n, hq, dh))
    P_prev = rng.normal(size=(K, hq, n)) * 2
    plog, kl, keys = O.proxy_drift(zq, Kc, Vc, P_prev, act, blk)
    assert np.array_equal(keys, np.arange(blk, blk + Bk))
    qt = torch.tensor(zq).permute(1, 0, 2)                                  # [Hq, K, dh]
    kt = torch.tensor(Kc[keys]).permute(1, 2, 0)                            # [Hq, dh, B]
    scores = (qt @ kt / math.sqrt(dh)).permute(1, 0, 2)                      # [K, Hq, B]
    assert np.allclose(plog, scores.numpy(), rtol=1e-12, atol=1e-12)
    want = F.kl_div(torch.log_softmax(torch.tensor(P_prev[..., keys]), -1), torch.log_softmax(scores, -1),
                    reduction="none", log_target=True).sum(-1)
    assert np.allclose(kl, want.numpy(), rtol=1e-10, atol=1e-13)
    # keys outside the active block: no effect on the "active" reading, an effect on "all"
    K2, V2, P2 = Kc.copy(), Vc.copy(), P_prev.copy()
    out = np.setdiff1d(np.arange(n), keys)
    K2[out] = rng.normal(size=K2[out].shape)
    V2[out] = rng.normal(size=V2[out].shape)
    P2[..., out] = rng.normal(size=P2[..., out].shape)
    assert np.array_equal(O.proxy_drift(zq, K2, V2, P2, act, blk)[1], kl)
    assert not np.allclose(O.proxy_drift(zq, K2, V2, P2, full, blk)[1], O.proxy_drift(zq, Kc, Vc, P_prev, full, blk)[1])


# ---- most-attended-token cosine policy [§5 "Drift Measurement Policy", Fig. 6(a)] ----------

def test_attended_token_change_planted_tokens_and_scores():
    """Queries aligned with one key recover that key as the most-attended token; the score is
    0 for an unchanged or rescaled key, 2 for a negated one, 1 for an orthogonal or zero one."""
    rng = np.random.default_rng(11)
    n, hq, hkv, dh = 7, 4, 2, 8
    K = rng.normal(size=(n, hkv, dh))
    targets = [2, 5, 0, 6, 3]
    q = np.zeros((len(targets), hq, dh))
    for r, j in enumerate(targets):
        for h in range(hq):
            q[r, h] = 40.0 * K[j, (h * hkv) // hq]
    Kref = K.copy()
    Kref[5] = -K[5]                       # negated: cos -1
    Kref[0] = 3.0 * K[0]                  # rescaled: cos 1
    e = np.zeros(dh)
    e[0] = 1.0
    Kref[6, 0] = e * np.linalg.norm(K[6, 0])
    Kref[6, 0] -= np.dot(Kref[6, 0], K[6, 0]) / np.dot(K[6, 0], K[6, 0]) * K[6, 0]   # orthogonal in head 0
    Kref[6, 1] = 0.0                      # zero row in head 1: cosine 0
    Kref[3] = -K[3]
    Kref[3, 1] = K[3, 1]                  # head 0 negated, head 1 unchanged: mean cos 0
    j, s, A = O.attended_token_change(q, K, Kref, hq, hkv)
    assert j.tolist() == targets
    assert np.allclose(A.sum(axis=1), 1.0)
    assert s[0] == pytest.approx(0.0, abs=1e-12)          # position 2 unchanged
    assert s[1] == pytest.approx(2.0, abs=1e-12)          # position 5 negated
    assert s[2] == pytest.approx(0.0, abs=1e-12)          # position 0 rescaled
    assert s[3] == pytest.approx(1.0, abs=1e-12)          # position 6: cos 0 and 0
    assert s[4] == pytest.approx(1.0, abs=1e-12)          # position 3: cos -1 and 1


def test_attended_token_change_ties_and_head_map():
    """Equal keys at two positions tie exactly and the lower position wins; all-zero keys give a
    uniform distribution (position 0); the query head -> KV head map is h * hkv // hq (grouped)."""
    rng = np.random.default_rng(12)
    n, hq, hkv, dh = 6, 4, 2, 4
    K = rng.normal(size=(n, hkv, dh)) * 0.01
    K[1] = rng.normal(size=(hkv, dh))
    K[4] = K[1]
    q = np.zeros((1, hq, dh))
    for h in range(hq):
        q[0, h] = 30.0 * K[1, (h * hkv) // hq] / np.linalg.norm(K[1, (h * hkv) // hq]) ** 2
    j, _, A = O.attended_token_change(q, K, K, hq, hkv)
    assert A[0, 1] == A[0, 4] and j[0] == 1
    j0, _, A0 = O.attended_token_change(q, np.zeros_like(K), K, hq, hkv)
    assert np.allclose(A0, 1.0 / n) and j0[0] == 0
    # grouped map: heads 0, 1 read KV head 0 (which points at position 2), heads 2, 3 read KV
    # head 1 (position 3, weaker); an interleaved map (h % hkv) would pair differently
    K = np.zeros((n, hkv, dh))
    K[2, 0, 0] = 1.0
    K[3, 1, 1] = 1.0
    q = np.zeros((1, hq, dh))
    q[0, 0, 0] = q[0, 1, 0] = 20.0        # heads 0, 1: strongly on position 2 through KV head 0
    q[0, 2, 1] = q[0, 3, 1] = 2.0         # heads 2, 3: weakly on position 3 through KV head 1
    j, _, A = O.attended_token_change(q, K, K, hq, hkv)
    assert j[0] == 2 and A[0, 2] > 0.49
    # the interleaved reading: heads 0 and 2 on KV head 0, heads 1 and 3 on KV head 1
    qi = q.copy()
    qi[0, 1], qi[0, 2] = q[0, 2], q[0, 1]
    ji, _, Ai = O.attended_token_change(qi, K, K, hq, hkv)
    assert not np.allclose(Ai, A)
