"""The C ABI without a GPU: the library loads, exports what include/polestar.h
declares, validates arguments on the host (no kernel launched), and its host
NVFP4 encoder agrees bit for bit with the oracle's codec."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from drift_driven_sparse_amd import binding as B
from oracle import polestar_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "polestar.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(polestar_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    declared = _declared_functions()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTED) == declared


def _dims(**kw):
    base = dict(d=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=768, n_pos=320, batch=1, block=32,
                win_prefix=64, win_suffix=32, n_clusters=8, top_k=4, vocab=0, dtype=B.F32, resid_fmt=B.RESID_RAW)
    base.update(kw)
    return B.Dims(**base)


def _params(**kw):
    base = dict(rms_eps=1e-6, tau_s=0.9, tau_suf=0.9, alpha=10.0, hist=5, mask_id=0, kmeans_iters=10)
    base.update(kw)
    return B.Params(**base)


def test_create_accepts_the_five_workload_shapes():
    shapes = [
        _dims(),
        _dims(d=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn=12288, n_pos=768, dtype=B.BF16),
        _dims(d=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn=12288, n_pos=1024, dtype=B.BF16),
        _dims(d=3584, n_heads=28, n_kv_heads=4, head_dim=128, ffn=18944, n_pos=640, dtype=B.BF16),
        _dims(d=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn=12288, n_pos=768, batch=16, vocab=126464,
              dtype=B.BF16, resid_fmt=B.RESID_NVFP4),
        # sweep shapes past one 192-row projection slab and 1024 positions
        _dims(d=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=512, n_pos=512, block=64, win_prefix=128,
              win_suffix=64, dtype=B.BF16),
        _dims(d=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=512, n_pos=4096, block=64, win_prefix=192,
              win_suffix=64, n_clusters=16, top_k=8, dtype=B.BF16),
    ]
    for dm in shapes:
        h = B.polestar_create(dm, _params(mask_id=max(dm.vocab - 1, 0)))
        assert B.polestar_workspace_size(h) > 0
        B.polestar_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(n_clusters=17, top_k=4), B.E_UNSUPPORTED),
    (dict(top_k=9), B.E_UNSUPPORTED),
    (dict(head_dim=96), B.E_UNSUPPORTED),
    (dict(n_heads=6, n_kv_heads=4), B.E_SHAPE),
    (dict(dtype=7), B.E_DTYPE),
    (dict(resid_fmt=9), B.E_DTYPE),
    (dict(resid_fmt=B.RESID_NVFP4), B.E_UNSUPPORTED),       # NVFP4 needs bf16 storage
    (dict(d=0), B.E_SHAPE),
    (dict(n_pos=16), B.E_SHAPE),
    (dict(win_prefix=224, win_suffix=64), B.E_UNSUPPORTED),  # window of more than 256 rows
    (dict(dtype=B.BF16, n_pos=8192), B.E_UNSUPPORTED),        # more than 4096 positions
    (dict(n_pos=2048), B.E_UNSUPPORTED),                      # float32 storage: at most 1024 positions
    (dict(dtype=B.BF16, d=200), B.E_UNSUPPORTED),
])
def test_create_rejects_bad_dims(kw, code):
    with pytest.raises(B.PolestarError) as e:
        B.polestar_create(_dims(**kw), _params())
    assert e.value.code == code


def test_calls_validate_before_launching():
    h = B.polestar_create(_dims(), _params())
    try:
        ws_bytes = B.polestar_workspace_size(h)
        L = B.Layer()
        sel = B.Packet()
        lib = B.lib()
        # NULL workspace / too small workspace / misaligned workspace: rejected on the host
        assert lib.polestar_cluster(h, B.CLUSTER_UPDATE, C.byref(L), 64, None, None, None, None, None, ws_bytes,
                                    None) == B.E_NULL
        assert lib.polestar_cluster(h, B.CLUSTER_UPDATE, C.byref(L), 64, None, None, None, None, 4096,
                                    ws_bytes - 1, None) == B.E_WORKSPACE
        assert lib.polestar_cluster(h, B.CLUSTER_UPDATE, C.byref(L), 64, None, None, None, None, 4096 + 16,
                                    ws_bytes, None) == B.E_ALIGN
        # missing window buffers
        assert lib.polestar_cluster(h, B.CLUSTER_UPDATE, C.byref(L), 64, None, None, None, None, 4096,
                                    ws_bytes, None) == B.E_NULL
        # block start outside the sequence
        L.win_h = L.win_z = L.win_m = 4096
        assert lib.polestar_cluster(h, B.CLUSTER_UPDATE, C.byref(L), 300, None, None, None, None, 4096,
                                    ws_bytes, None) == B.E_ARG
        assert lib.polestar_cluster(h, 5, C.byref(L), 64, None, None, None, None, 4096, ws_bytes, None) == B.E_ARG
        # drift without a selection packet / with delta but no logits
        assert lib.polestar_drift(h, B.DRIFT_REFRESH, C.byref(L), 64, 4096, None, None, None, None, None, None,
                                  4096, ws_bytes, None) == B.E_NULL
        sel.idx = sel.count = 4096
        assert lib.polestar_drift(h, B.DRIFT_REFRESH, C.byref(L), 64, 4096, None, None, None, C.byref(sel), None,
                                  4096, 4096, ws_bytes, None) == B.E_NULL
        # a query cache needs its validity flags and 16-byte alignment
        Lq = B.Layer(w_qkv=4096, k_cache=4096, v_cache=4096, win_z=4096, win_m=4096, proxy_logits=4096, q_win=4096)
        assert lib.polestar_drift(h, B.DRIFT_REFRESH, C.byref(Lq), 64, 4096, None, None, None, C.byref(sel), None,
                                  None, 4096, ws_bytes, None) == B.E_NULL
        Lq.q_ok, Lq.q_win = 4096, 4096 + 8
        assert lib.polestar_drift(h, B.DRIFT_REFRESH, C.byref(Lq), 64, 4096, None, None, None, C.byref(sel), None,
                                  None, 4096, ws_bytes, None) == B.E_ALIGN
        # refresh with a misaligned weight
        L.w_o, L.w_gu, L.w_down = 4096 + 2, 4096, 4096
        assert lib.polestar_refresh(h, C.byref(L), 64, 4096, C.byref(sel), None, None, None, 4096, 4096, 4096,
                                    ws_bytes, None) == B.E_ALIGN
        # block entry: missing inputs, an unknown mode, a missing layer buffer, overlapping rows
        entry = lib.polestar_entry
        assert entry(h, B.ENTRY_FULL, C.byref(L), 64, None, 4096, 8192, None, None, 4096, ws_bytes, None) == B.E_NULL
        assert entry(h, 7, C.byref(L), 64, 4096, 4096, 1 << 30, None, None, 4096, ws_bytes, None) == B.E_ARG
        assert entry(h, B.ENTRY_WINDOW, C.byref(L), 300, 4096, 4096, 1 << 30, None, None, 4096, ws_bytes,
                     None) == B.E_ARG
        L.w_o = 4096
        L.w_qkv = L.k_cache = L.v_cache = L.proxy_logits = 4096
        assert entry(h, B.ENTRY_FULL, C.byref(L), 64, 4096, 4096, 1 << 30, None, None, 4096, ws_bytes - 1,
                     None) == B.E_WORKSPACE
        L.w_qkv = 4096 + 8
        assert entry(h, B.ENTRY_FULL, C.byref(L), 64, 4096, 4096, 1 << 30, None, None, 4096, ws_bytes, None) == B.E_ALIGN
        L.w_qkv = 4096
        L.proxy_logits = None
        assert entry(h, B.ENTRY_FULL, C.byref(L), 64, 4096, 4096, 1 << 30, None, None, 4096, ws_bytes, None) == B.E_NULL
        L.proxy_logits = 4096
        rows_bytes = 320 * 256 * 4
        assert entry(h, B.ENTRY_FULL, C.byref(L), 64, 1 << 20, 4096, (1 << 20) + rows_bytes - 16, None, None, 4096,
                     ws_bytes, None) == B.E_ARG
        assert entry(h, B.ENTRY_FULL, C.byref(L), 64, (1 << 20) + rows_bytes - 16, 4096, 1 << 20, None, None, 4096,
                     ws_bytes, None) == B.E_ARG
        # the whole-stack step: layer count, mode, and every layer validated before any launch
        pk = B.Packet(rows=4096, idx=4096, count=4096)
        arr = (B.Layer * 2)(B.Layer(), B.Layer())
        step = lib.polestar_step
        assert step(h, B.DRIFT_REFRESH, 0, arr, 64, 4096, 4096, C.byref(pk), C.byref(pk), None, None, None, None,
                    4096, ws_bytes, None) == B.E_ARG
        assert step(h, 9, 2, arr, 64, 4096, 4096, C.byref(pk), C.byref(pk), None, None, None, None, 4096, ws_bytes,
                    None) == B.E_ARG
        assert step(h, B.DRIFT_REFRESH, 2, None, 64, 4096, 4096, C.byref(pk), C.byref(pk), None, None, None, None,
                    4096, ws_bytes, None) == B.E_NULL
        assert step(h, B.DRIFT_ACTIVE_ONLY, 2, arr, 64, 4096, 4096, C.byref(pk), C.byref(pk), None, None, None,
                    None, 4096, ws_bytes, None) == B.E_NULL      # layers without weights
        # the entry commit needs its outputs and a vocabulary
        assert lib.polestar_entry_commit(h, 64, 4096, 4096, 4096, 4096, None, 4096, 4096, 4096, 4096, 4096,
                                         ws_bytes, None) == B.E_NULL
        assert lib.polestar_entry_commit(h, 64, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096,
                                         ws_bytes, None) == B.E_SHAPE
        # commit needs a vocabulary
        assert lib.polestar_commit(h, 64, 4096, 4096, None, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096,
                                   4096, 4096, 4096, ws_bytes, None) == B.E_SHAPE
        # weight kinds
        with pytest.raises(B.PolestarError):
            B.polestar_weight_packed_size(h, 99)
        with pytest.raises(B.PolestarError):
            B.polestar_weight_packed_size(h, B.W_LM)
        assert B.polestar_weight_packed_size(h, B.W_QKV) == (4 + 8) * 64 * 256 * 4
    finally:
        B.polestar_destroy(h)


def test_should_refresh_matches_oracle():
    for tau in (0, 1, 3, 4):
        for c in range(8):
            assert B.polestar_should_refresh(c, tau) == O.should_refresh(c, tau)
    assert not B.polestar_should_refresh(10**6, -1)


def test_host_nvfp4_encoder_matches_oracle():
    rng = np.random.default_rng(11)
    rows, d = 64, 256
    x = (rng.normal(size=(rows, d)) * np.exp(rng.uniform(-12, 8, size=(rows, 1)))).astype(np.float32)
    # exact ties of E2M1 and E4M3 boundaries
    x[0, :16] = np.float32([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -5, 0, -0.0, 4, 3, 2])
    x[1, :16] = 0.0
    x[2, :16] = np.float32(448 * 6 * 4)              # saturating scale
    x[3, :16] = np.float32(2.0 ** -12)               # subnormal scale
    codes = np.zeros((rows, d // 2), np.uint8)
    scales = np.zeros((rows, d // 16), np.uint8)
    B.polestar_nvfp4_pack_host(x.ctypes.data, rows, d, codes.ctypes.data, scales.ctypes.data)
    oc, os_ = O.nvfp4_quantize(x)
    assert np.array_equal(scales, os_)
    assert np.array_equal(codes, oc)


def test_residual_format_sizes_and_rejections():
    # bytes per row [App. C.3; Table 11]: nibbles + E4M3 per 16, E4M3 bytes, int8 + E8M0 per 32,
    # nibbles + E8M0 per 32
    assert B.polestar_resid_bytes(B.RESID_NVFP4, 4096) == (2048, 256)
    assert B.polestar_resid_bytes(B.RESID_FP8, 4096) == (4096, 0)
    assert B.polestar_resid_bytes(B.RESID_MXINT8, 4096) == (4096, 128)
    assert B.polestar_resid_bytes(B.RESID_MXFP4, 3584) == (1792, 112)
    assert B.polestar_resid_bytes(B.RESID_RAW, 256) == (0, 0)
    lib = B.lib()
    cb, sb = C.c_int64(), C.c_int64()
    assert lib.polestar_resid_bytes(7, 256, C.byref(cb), C.byref(sb)) == B.E_DTYPE
    assert lib.polestar_resid_bytes(B.RESID_FP8, 48, C.byref(cb), C.byref(sb)) == B.E_SHAPE
    assert lib.polestar_resid_pack(B.RESID_RAW, None, 1, 32, None, None, None) == B.E_DTYPE
    assert lib.polestar_resid_pack(B.RESID_MXFP4, None, 1, 32, None, None, None) == B.E_NULL
    assert lib.polestar_resid_unpack(B.RESID_MXINT8, None, None, 1, 40, None, None) == B.E_SHAPE
    # residual formats need bf16 storage; unknown formats are a dtype error
    h = C.c_void_p()
    for fmt in (B.RESID_FP8, B.RESID_MXINT8, B.RESID_MXFP4):
        assert lib.polestar_create(C.byref(_dims(resid_fmt=fmt)), C.byref(_params()), C.byref(h)) == B.E_UNSUPPORTED
    assert lib.polestar_create(C.byref(_dims(resid_fmt=9)), C.byref(_params()), C.byref(h)) == B.E_DTYPE


def test_step_noalloc_rejects_a_workspace_beyond_the_scratch():
    """polestar_step_noalloc returns E_SCRATCH, before any HIP call, for a handle whose workspace
    exceeds the static scratch (the batch-16 LLaDA-shaped workload needs about 1 GiB); the
    LLaDA-shaped stack of one sequence fits."""
    lib = B.lib()
    big = B.polestar_create(_dims(d=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn=12288, n_pos=768, batch=16,
                                  vocab=126464, dtype=B.BF16, resid_fmt=B.RESID_NVFP4), _params(mask_id=126463))
    one = B.polestar_create(_dims(d=4096, n_heads=32, n_kv_heads=32, head_dim=128, ffn=12288, n_pos=1024,
                                  dtype=B.BF16), _params())
    try:
        assert B.polestar_workspace_size(big) > B.SCRATCH_BYTES
        assert B.polestar_workspace_size(one) <= B.SCRATCH_BYTES
        L = (B.Layer * 1)()
        pk = B.Packet(rows=4096, idx=4096, count=4096)
        rc = lib.polestar_step_noalloc(big, B.DRIFT_REFRESH, 1, L, 512, 4096, 4096, C.byref(pk), C.byref(pk), None,
                                       None, None, None, None)
        assert rc == B.E_SCRATCH
        assert "static scratch" in B.strerror(rc)
        assert lib.polestar_step_noalloc(None, 0, 1, L, 0, 0, 0, None, None, None, None, None, None, None) == B.E_NULL
    finally:
        B.polestar_destroy(big)
        B.polestar_destroy(one)
