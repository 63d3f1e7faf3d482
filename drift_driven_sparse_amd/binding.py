"""ctypes binding of libpolestar.so (include/polestar.h): argument marshalling only.

Every refresh-path step runs in the library's HIP kernels; this module converts
Python/torch arguments into the C structs and pointers the library takes.  It
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpolestar.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUPPORTED, E_WORKSPACE, E_ALIGN, E_HIP, E_ARG = 0, -1, -2, -3, -4, -5, -6, -7, -8
E_SCRATCH = -9
SCRATCH_BYTES = 192 << 20
F32, BF16 = 0, 1
RESID_RAW, RESID_NVFP4, RESID_FP8, RESID_MXINT8, RESID_MXFP4 = 0, 1, 2, 3, 4
RESID_BY_NAME = {"raw": RESID_RAW, "nvfp4": RESID_NVFP4, "fp8": RESID_FP8, "mxint8": RESID_MXINT8,
                 "mxfp4": RESID_MXFP4}
CLUSTER_ENTRY, CLUSTER_UPDATE = 0, 1
DRIFT_REFRESH, DRIFT_ACTIVE_ONLY = 0, 1
ENTRY_FULL, ENTRY_WINDOW = 0, 1
PROXY_ALL, PROXY_ACTIVE = 0, 1
W_QKV, W_O, W_GU, W_DOWN, W_KV, W_LM = 0, 1, 2, 3, 4, 5

EXPORTED = [
    "polestar_create", "polestar_destroy", "polestar_strerror", "polestar_workspace_size",
    "polestar_set_check", "polestar_weight_packed_size", "polestar_pack_weight", "polestar_cluster",
    "polestar_drift", "polestar_refresh", "polestar_commit", "polestar_should_refresh",
    "polestar_nvfp4_pack", "polestar_nvfp4_unpack", "polestar_nvfp4_pack_host", "polestar_profile",
    "polestar_profile_read", "polestar_resid_bytes", "polestar_resid_pack", "polestar_resid_unpack",
    "polestar_kv_staleness", "polestar_attended_change", "polestar_entry", "polestar_entry_commit", "polestar_step", "polestar_step_noalloc",
]
KERNELS = ["cluster", "prep", "qkv", "attn", "topk", "oproj", "oreduce", "gu", "down", "dreduce", "kvnext",
           "lmprep", "lmhead", "decide", "kl"]


class Dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "d", "n_heads", "n_kv_heads", "head_dim", "ffn", "n_pos", "batch", "block", "win_prefix",
        "win_suffix", "n_clusters", "top_k", "vocab", "dtype", "resid_fmt")]


class Params(C.Structure):
    _fields_ = [("rms_eps", C.c_float), ("tau_s", C.c_float), ("tau_suf", C.c_float), ("alpha", C.c_float),
                ("hist", C.c_int32), ("mask_id", C.c_int32), ("kmeans_iters", C.c_int32),
                ("proxy_support", C.c_int32)]


class Layer(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("w_gu", C.c_void_p), ("w_down", C.c_void_p),
                ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("win_h", C.c_void_p),
                ("win_codes", C.c_void_p), ("win_scales", C.c_void_p), ("win_z", C.c_void_p),
                ("win_m", C.c_void_p), ("proxy_logits", C.c_void_p), ("q_win", C.c_void_p), ("q_ok", C.c_void_p)]


class Packet(C.Structure):
    _fields_ = [("rows", C.c_void_p), ("idx", C.c_void_p), ("count", C.c_void_p)]


class Check(C.Structure):
    _fields_ = [("qkv", C.c_void_p), ("attn_out", C.c_void_p), ("hp", C.c_void_p), ("out", C.c_void_p),
                ("kv_next", C.c_void_p)]


_lib: Optional[C.CDLL] = None


class PolestarError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m drift_driven_sparse_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.polestar_create.argtypes = [C.POINTER(Dims), C.POINTER(Params), C.POINTER(vp)]
        L.polestar_destroy.argtypes = [vp]
        L.polestar_destroy.restype = None
        L.polestar_strerror.argtypes = [C.c_int]
        L.polestar_strerror.restype = C.c_char_p
        L.polestar_workspace_size.argtypes = [vp, C.POINTER(sz)]
        L.polestar_set_check.argtypes = [vp, C.POINTER(Check)]
        L.polestar_weight_packed_size.argtypes = [vp, C.c_int, C.POINTER(sz)]
        L.polestar_pack_weight.argtypes = [vp, C.c_int, vp, vp, vp]
        L.polestar_cluster.argtypes = [vp, C.c_int, C.POINTER(Layer), i32, C.POINTER(Packet), vp, vp, vp, vp, sz, vp]
        L.polestar_entry.argtypes = [vp, C.c_int, C.POINTER(Layer), i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.polestar_step.argtypes = [vp, C.c_int, i32, C.POINTER(Layer), i32, vp, vp, C.POINTER(Packet),
                                    C.POINTER(Packet), vp, vp, vp, vp, vp, sz, vp]
        L.polestar_step_noalloc.argtypes = [vp, C.c_int, i32, C.POINTER(Layer), i32, vp, vp, C.POINTER(Packet),
                                            C.POINTER(Packet), vp, vp, vp, vp, vp]
        L.polestar_entry_commit.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.polestar_drift.argtypes = [vp, C.c_int, C.POINTER(Layer), i32, vp, C.POINTER(Packet), vp, vp,
                                     C.POINTER(Packet), vp, vp, vp, sz, vp]
        L.polestar_refresh.argtypes = [vp, C.POINTER(Layer), i32, vp, C.POINTER(Packet), vp, vp, vp, vp, vp, vp, sz, vp]
        L.polestar_commit.argtypes = [vp, i32, vp, vp, C.POINTER(Packet), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
        L.polestar_should_refresh.argtypes = [i32, i32]
        L.polestar_nvfp4_pack.argtypes = [vp, i64, i32, vp, vp, vp]
        L.polestar_nvfp4_unpack.argtypes = [vp, vp, i64, i32, vp, vp]
        L.polestar_nvfp4_pack_host.argtypes = [vp, i64, i32, vp, vp]
        L.polestar_resid_bytes.argtypes = [i32, i32, C.POINTER(i64), C.POINTER(i64)]
        L.polestar_resid_pack.argtypes = [i32, vp, i64, i32, vp, vp, vp]
        L.polestar_resid_unpack.argtypes = [i32, vp, vp, i64, i32, vp, vp]
        L.polestar_kv_staleness.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.polestar_attended_change.argtypes = [vp, vp, i32, i32, C.c_int64, vp, vp, vp, vp, vp]
        L.polestar_profile.argtypes = [vp, C.c_int]
        L.polestar_profile_read.argtypes = [vp, C.POINTER(C.c_double), C.POINTER(i32)]
        for name in EXPORTED:
            f = getattr(L, name)
            if name not in ("polestar_destroy", "polestar_strerror"):
                f.restype = C.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().polestar_strerror(code).decode()


def _ck(code: int, where: str) -> None:
    if code != OK:
        raise PolestarError(code, where)


def ptr(t) -> Optional[int]:
    """Device/host address of a tensor (None passes NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_ptr(stream=None) -> Optional[int]:
    import torch
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ---- thin wrappers with the C names ------------------------------------------------------
def polestar_create(dims: Dims, params: Params) -> int:
    h = C.c_void_p()
    _ck(lib().polestar_create(C.byref(dims), C.byref(params), C.byref(h)), "polestar_create")
    return h.value


def polestar_destroy(h: int) -> None:
    lib().polestar_destroy(h)


def polestar_workspace_size(h: int) -> int:
    n = C.c_size_t()
    _ck(lib().polestar_workspace_size(h, C.byref(n)), "polestar_workspace_size")
    return n.value


def polestar_set_check(h: int, chk: Optional[Check]) -> None:
    _ck(lib().polestar_set_check(h, C.byref(chk) if chk is not None else None), "polestar_set_check")


def polestar_weight_packed_size(h: int, which: int) -> int:
    n = C.c_size_t()
    _ck(lib().polestar_weight_packed_size(h, which, C.byref(n)), "polestar_weight_packed_size")
    return n.value


def polestar_pack_weight(h: int, which: int, src, dst, stream=None) -> None:
    _ck(lib().polestar_pack_weight(h, which, ptr(src), ptr(dst), stream_ptr(stream)), "polestar_pack_weight")


def _pk(p: Optional[Packet]):
    return C.byref(p) if p is not None else None


def polestar_cluster(h, mode, layer: Layer, blk_start, u_in: Optional[Packet], init_idx, entry_h, objective,
                     ws, ws_bytes, stream=None) -> None:
    _ck(lib().polestar_cluster(h, mode, C.byref(layer), blk_start, _pk(u_in), ptr(init_idx), ptr(entry_h),
                               ptr(objective), ptr(ws), ws_bytes, stream_ptr(stream)), "polestar_cluster")


def polestar_drift(h, mode, layer: Layer, blk_start, h_active, u_in: Optional[Packet], D, topk, sel: Packet,
                   act_logits, delta, ws, ws_bytes, stream=None) -> None:
    _ck(lib().polestar_drift(h, mode, C.byref(layer), blk_start, ptr(h_active), _pk(u_in), ptr(D), ptr(topk),
                             C.byref(sel), ptr(act_logits), ptr(delta), ptr(ws), ws_bytes, stream_ptr(stream)),
        "polestar_drift")


def polestar_refresh(h, layer: Layer, blk_start, h_active, sel: Packet, w_kv_next, k_next, v_next, h_active_out,
                     u_rows, ws, ws_bytes, stream=None) -> None:
    _ck(lib().polestar_refresh(h, C.byref(layer), blk_start, ptr(h_active), C.byref(sel), ptr(w_kv_next),
                               ptr(k_next), ptr(v_next), ptr(h_active_out), ptr(u_rows), ptr(ws), ws_bytes,
                               stream_ptr(stream)), "polestar_refresh")


def polestar_entry(h, mode, layer: Layer, blk_start, h_in, init_idx, h_out, objective, act_logits, ws, ws_bytes,
                   stream=None) -> None:
    _ck(lib().polestar_entry(h, mode, C.byref(layer), blk_start, ptr(h_in), ptr(init_idx), ptr(h_out),
                             ptr(objective), ptr(act_logits), ptr(ws), ws_bytes, stream_ptr(stream)),
        "polestar_entry")


def polestar_entry_commit(h, blk_start, w_lm, h_full, active_masked, suffix_masked, commit_active, commit_suffix,
                          conf_active, yhat_active, conf_suffix, ws, ws_bytes, stream=None) -> None:
    _ck(lib().polestar_entry_commit(h, blk_start, ptr(w_lm), ptr(h_full), ptr(active_masked), ptr(suffix_masked),
                                    ptr(commit_active), ptr(commit_suffix), ptr(conf_active), ptr(yhat_active),
                                    ptr(conf_suffix), ptr(ws), ws_bytes, stream_ptr(stream)),
        "polestar_entry_commit")


def polestar_step(h, mode, layers, blk_start, h_act0, h_act1, pk0: Packet, pk1: Packet, D, topk, act_logits, delta,
                  ws, ws_bytes, stream=None) -> None:
    arr = (Layer * len(layers))(*layers)
    _ck(lib().polestar_step(h, mode, len(layers), arr, blk_start, ptr(h_act0), ptr(h_act1), C.byref(pk0),
                            C.byref(pk1), ptr(D), ptr(topk), ptr(act_logits), ptr(delta), ptr(ws), ws_bytes,
                            stream_ptr(stream)), "polestar_step")


def polestar_step_noalloc(h, mode, layers, blk_start, h_act0, h_act1, pk0: Packet, pk1: Packet, D, topk, act_logits,
                          delta, stream=None) -> None:
    arr = (Layer * len(layers))(*layers)
    _ck(lib().polestar_step_noalloc(h, mode, len(layers), arr, blk_start, ptr(h_act0), ptr(h_act1), C.byref(pk0),
                                    C.byref(pk1), ptr(D), ptr(topk), ptr(act_logits), ptr(delta), stream_ptr(stream)),
        "polestar_step_noalloc")


def polestar_commit(h, blk_start, w_lm, h_final, u_final: Optional[Packet], delta, active_masked, suffix_masked,
                    hist_vals, hist_cnt, commit_active, commit_suffix, conf_active, yhat_active, spike, conf_suffix,
                    ws, ws_bytes, stream=None) -> None:
    _ck(lib().polestar_commit(h, blk_start, ptr(w_lm), ptr(h_final), _pk(u_final), ptr(delta), ptr(active_masked),
                              ptr(suffix_masked), ptr(hist_vals), ptr(hist_cnt), ptr(commit_active),
                              ptr(commit_suffix), ptr(conf_active), ptr(yhat_active), ptr(spike), ptr(conf_suffix),
                              ptr(ws), ws_bytes, stream_ptr(stream)), "polestar_commit")


def polestar_should_refresh(decoded_since_refresh: int, tau_upd: int) -> bool:
    return bool(lib().polestar_should_refresh(decoded_since_refresh, tau_upd))


def polestar_nvfp4_pack(x, rows, d, codes, scales, stream=None) -> None:
    _ck(lib().polestar_nvfp4_pack(ptr(x), rows, d, ptr(codes), ptr(scales), stream_ptr(stream)), "polestar_nvfp4_pack")


def polestar_nvfp4_unpack(codes, scales, rows, d, x, stream=None) -> None:
    _ck(lib().polestar_nvfp4_unpack(ptr(codes), ptr(scales), rows, d, ptr(x), stream_ptr(stream)),
        "polestar_nvfp4_unpack")


def polestar_resid_bytes(fmt: int, d: int) -> Tuple[int, int]:
    cb, sb = C.c_int64(), C.c_int64()
    _ck(lib().polestar_resid_bytes(fmt, d, C.byref(cb), C.byref(sb)), "polestar_resid_bytes")
    return cb.value, sb.value


def polestar_resid_pack(fmt, x, rows, d, codes, scales, stream=None) -> None:
    _ck(lib().polestar_resid_pack(fmt, ptr(x), rows, d, ptr(codes), ptr(scales), stream_ptr(stream)),
        "polestar_resid_pack")


def polestar_resid_unpack(fmt, codes, scales, rows, d, x, stream=None) -> None:
    _ck(lib().polestar_resid_unpack(fmt, ptr(codes), ptr(scales), rows, d, ptr(x), stream_ptr(stream)),
        "polestar_resid_unpack")


def polestar_attended_change(h: int, q, rows: int, q_ld: int, q_bstride: int, k_cache, k_ref, top_pos, score,
                             stream=None) -> None:
    _ck(lib().polestar_attended_change(h, ptr(q), rows, q_ld, q_bstride, ptr(k_cache), ptr(k_ref), ptr(top_pos),
                                       ptr(score), stream_ptr(stream)), "polestar_attended_change")


def polestar_kv_staleness(h: int, k_cache, v_cache, k_ref, v_ref, stale, stream=None) -> None:
    _ck(lib().polestar_kv_staleness(h, ptr(k_cache), ptr(v_cache), ptr(k_ref), ptr(v_ref), ptr(stale),
                                    stream_ptr(stream)), "polestar_kv_staleness")


def polestar_nvfp4_pack_host(x, rows, d, codes, scales) -> None:
    _ck(lib().polestar_nvfp4_pack_host(ptr(x), rows, d, ptr(codes), ptr(scales)), "polestar_nvfp4_pack_host")


def polestar_profile(h: int, enable: bool) -> None:
    _ck(lib().polestar_profile(h, 1 if enable else 0), "polestar_profile")


def polestar_profile_read(h: int):
    """{kernel name: (total ms, launches)} of the recorded launches."""
    n = len(KERNELS)
    ms = (C.c_double * n)()
    cnt = (C.c_int32 * n)()
    _ck(lib().polestar_profile_read(h, ms, cnt), "polestar_profile_read")
    return {KERNELS[i]: (ms[i], cnt[i]) for i in range(n)}
