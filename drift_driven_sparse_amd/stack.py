"""Device state of a refresh-path layer stack and its per-step layer loop.

Every step of the method runs in the HIP library; this module owns the device
buffers (PyTorch allocations) and issues the C-ABI calls layer by layer:

  refresh step, layer l:  polestar_cluster(UPDATE, packet U(t,l))
                          polestar_drift(REFRESH)  -> S_l
                          polestar_refresh         -> U(t,l+1), next active rows
  step without refresh:   polestar_drift(ACTIVE_ONLY) + polestar_refresh (active rows only)

The update packet of layer l is consumed by layer l+1 (its window rows are
patched and its K/V rows for S_l are recomputed from U), so packets and
active rows alternate between two buffers.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import binding as B

_TDT = {B.F32: torch.float32, B.BF16: torch.bfloat16}


class RefreshStack:
    def __init__(self, dims: B.Dims, params: B.Params, n_layers: int, device="cuda", q_cache: bool = True):
        self.dims, self.params, self.n_layers, self.device = dims, params, n_layers, device
        self.h = B.polestar_create(dims, params)
        self.ws_bytes = B.polestar_workspace_size(self.h)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        d, bt, n = dims.d, dims.batch, dims.n_pos
        self.win_max = dims.win_prefix + dims.win_suffix
        self.tdt = _TDT[dims.dtype]
        self.resid = dims.resid_fmt != B.RESID_RAW   # window rows stored as residual codes
        cb, sb = B.polestar_resid_bytes(dims.resid_fmt, dims.d) if self.resid else (0, 0)
        kvd = dims.n_kv_heads * dims.head_dim
        self.layers: List[Dict[str, torch.Tensor]] = []
        for _ in range(n_layers):
            L = {
                "k_cache": torch.zeros(bt, n, dims.n_kv_heads, dims.head_dim, dtype=self.tdt, device=device),
                "v_cache": torch.zeros(bt, dims.n_kv_heads, dims.head_dim, n, dtype=self.tdt, device=device),
                "win_z": torch.zeros(bt, dims.n_clusters, d, dtype=self.tdt, device=device),
                "win_m": torch.zeros(bt, self.win_max, dtype=torch.int32, device=device),
                "proxy_logits": torch.zeros(bt, dims.n_clusters, dims.n_heads, n, dtype=torch.float32, device=device),
            }
            if q_cache and dims.dtype == B.BF16 and not self.resid:   # window-row queries kept across steps
                L["q_win"] = torch.zeros(bt, self.win_max, dims.n_heads * dims.head_dim, dtype=torch.float32,
                                         device=device)
                L["q_ok"] = torch.zeros(bt, dtype=torch.int32, device=device)
            if self.resid:
                L["win_codes"] = torch.zeros(bt, self.win_max, cb, dtype=torch.uint8, device=device)
                L["win_scales"] = torch.zeros(bt, self.win_max, max(sb, 1), dtype=torch.uint8, device=device)
            else:
                L["win_h"] = torch.zeros(bt, self.win_max, d, dtype=self.tdt, device=device)
            self.layers.append(L)
        self.structs: List[Optional[B.Layer]] = [None] * n_layers
        # step buffers (two of each, alternating between layers)
        self.h_act = [torch.zeros(bt, dims.block, d, dtype=self.tdt, device=device) for _ in range(2)]
        self.pk_rows = [torch.zeros(bt, self.win_max, d, dtype=self.tdt, device=device) for _ in range(2)]
        self.pk_idx = [torch.zeros(bt, self.win_max, dtype=torch.int32, device=device) for _ in range(2)]
        self.pk_cnt = [torch.zeros(bt, dtype=torch.int32, device=device) for _ in range(2)]
        self.packets = [self._packet(i) for i in range(2)]
        self.D = torch.zeros(bt, dims.n_clusters, dtype=torch.float32, device=device)
        self.topk = torch.zeros(bt, dims.top_k, dtype=torch.int32, device=device)
        self.act_logits = torch.zeros(bt, dims.block, dims.n_heads, n, dtype=torch.float32, device=device)
        self.delta = torch.zeros(bt, dims.block, dtype=torch.float32, device=device)
        self.last_packet = 0
        self.h_seq: Optional[List[torch.Tensor]] = None   # block entry: layer inputs of every position

    def _packet(self, i: int) -> B.Packet:
        return B.Packet(rows=self.pk_rows[i].data_ptr(), idx=self.pk_idx[i].data_ptr(),
                        count=self.pk_cnt[i].data_ptr())

    def close(self):
        if self.h:
            B.polestar_destroy(self.h)
            self.h = None

    # ---- weights ----------------------------------------------------------------------------
    def _pack(self, which: int, src: torch.Tensor) -> torch.Tensor:
        n = B.polestar_weight_packed_size(self.h, which) // src.element_size()
        dst = torch.empty(n, dtype=src.dtype, device=self.device)
        B.polestar_pack_weight(self.h, which, src.contiguous(), dst)
        return dst

    def set_layer_weights(self, l: int, W: Dict[str, torch.Tensor]) -> None:
        """W: wq, wk, wv, wo, wg, wu, wd in [out, in] layout, storage dtype."""
        L = self.layers[l]
        L["w_qkv"] = self._pack(B.W_QKV, torch.cat([W["wq"], W["wk"], W["wv"]], 0))
        L["w_o"] = self._pack(B.W_O, W["wo"])
        L["w_gu"] = self._pack(B.W_GU, torch.cat([W["wg"], W["wu"]], 0))
        L["w_down"] = self._pack(B.W_DOWN, W["wd"])
        self.structs[l] = None

    def struct(self, l: int) -> B.Layer:
        if self.structs[l] is None:
            L = self.layers[l]
            s = B.Layer()
            for name in ("w_qkv", "w_o", "w_gu", "w_down", "k_cache", "v_cache", "win_h", "win_codes",
                         "win_scales", "win_z", "win_m", "proxy_logits", "q_win", "q_ok"):
                t = L.get(name)
                setattr(s, name, t.data_ptr() if t is not None else None)
            self.structs[l] = s
        return self.structs[l]

    # ---- block entry: clustering of the cached window rows ----------------------------------
    def block_entry(self, blk_start: int, entry_rows: List[torch.Tensor], init_idx: List[torch.Tensor]) -> None:
        """entry_rows[l]: window rows [batch, win_max, d]; init_idx[l]: [batch, K] int32."""
        for l in range(self.n_layers):
            B.polestar_cluster(self.h, B.CLUSTER_ENTRY, self.struct(l), blk_start, None, init_idx[l], entry_rows[l],
                               None, self.ws, self.ws_bytes)

    def entry_forward(self, blk_start: int, h0: torch.Tensor, init_idx: List[torch.Tensor], full: bool = True,
                      stream=None) -> torch.Tensor:
        """Block entry of every layer: h0 [batch, n_pos, d] is layer 0's input; each layer recomputes
        every position (full) or the window and the active block, clusters its window rows and sets
        its first drift reference; the last layer also sets the active block's logits, the first
        reference of the commit drift.  Returns the last layer's output rows."""
        if self.h_seq is None:
            shape = (self.dims.batch, self.dims.n_pos, self.dims.d)
            self.h_seq = [torch.empty(shape, dtype=self.tdt, device=self.device) for _ in range(2)]
        mode = B.ENTRY_FULL if full else B.ENTRY_WINDOW
        self.h_seq[0].copy_(h0)
        cur = 0
        for l in range(self.n_layers):
            last = l == self.n_layers - 1
            B.polestar_entry(self.h, mode, self.struct(l), blk_start, self.h_seq[cur], init_idx[l],
                             self.h_seq[1 - cur], None, self.act_logits if last else None, self.ws, self.ws_bytes,
                             stream)
            cur = 1 - cur
        return self.h_seq[cur]

    # ---- Polestar-Commit of the last layer's outputs ------------------------------------------
    def set_lm_head(self, w_lm: torch.Tensor) -> None:
        """W_lm [vocab, d] in the storage dtype; also allocates the commit state and outputs."""
        d, bt, Bk, suf = self.dims, self.dims.batch, self.dims.block, self.dims.win_suffix
        self.w_lm = self._pack(B.W_LM, w_lm)
        H = max(self.params.hist, 1)
        dev = self.device
        self.hist_vals = torch.zeros(bt, Bk, H, dtype=torch.float32, device=dev)
        self.hist_cnt = torch.zeros(bt, Bk, dtype=torch.int32, device=dev)
        self.active_masked = torch.ones(bt, Bk, dtype=torch.uint8, device=dev)
        self.suffix_masked = torch.ones(bt, max(suf, 1), dtype=torch.uint8, device=dev)
        self.commit_active = torch.zeros(bt, Bk, dtype=torch.uint8, device=dev)
        self.commit_suffix = torch.zeros(bt, max(suf, 1), dtype=torch.uint8, device=dev)
        self.conf_active = torch.zeros(bt, Bk, dtype=torch.float32, device=dev)
        self.yhat_active = torch.zeros(bt, Bk, dtype=torch.int32, device=dev)
        self.spike = torch.zeros(bt, Bk, dtype=torch.float32, device=dev)
        self.conf_suffix = torch.zeros(bt, max(suf, 1), dtype=torch.float32, device=dev)

    def commit(self, blk_start: int, h_final: torch.Tensor) -> None:
        """polestar_commit on the last step's outputs: its active rows h_final, its last layer's
        update packet and active drift delta."""
        B.polestar_commit(self.h, blk_start, self.w_lm, h_final, self.packets[self.last_packet], self.delta,
                          self.active_masked, self.suffix_masked, self.hist_vals, self.hist_cnt,
                          self.commit_active, self.commit_suffix, self.conf_active, self.yhat_active, self.spike,
                          self.conf_suffix, self.ws, self.ws_bytes)

    # ---- one denoising step -----------------------------------------------------------------
    def step(self, blk_start: int, h_in: torch.Tensor, refresh: bool = True, commit_delta: bool = True,
             per_layer: bool = False) -> torch.Tensor:
        """Runs every layer on the active rows h_in [batch, B, d]; returns the last layer's active rows.
        One polestar_step call for the whole stack, or with per_layer the cluster / drift / refresh
        calls of each layer (the same launches)."""
        self.h_act[0].copy_(h_in)
        mode = B.DRIFT_REFRESH if refresh else B.DRIFT_ACTIVE_ONLY
        if not per_layer:
            B.polestar_step(self.h, mode, [self.struct(l) for l in range(self.n_layers)], blk_start, self.h_act[0],
                            self.h_act[1], self.packets[0], self.packets[1], self.D, self.topk,
                            self.act_logits if commit_delta else None, self.delta if commit_delta else None,
                            self.ws, self.ws_bytes)
            self.last_packet = (self.n_layers - 1) % 2
            return self.h_act[self.n_layers % 2]
        cur_h = 0
        pk = 0
        u_in = None
        for l in range(self.n_layers):
            Ls = self.struct(l)
            last = l == self.n_layers - 1
            if refresh:
                B.polestar_cluster(self.h, B.CLUSTER_UPDATE, Ls, blk_start, u_in, None, None, None, self.ws,
                                   self.ws_bytes)
            sel = self.packets[pk]
            B.polestar_drift(self.h, mode, Ls, blk_start, self.h_act[cur_h], u_in, self.D, self.topk, sel,
                             self.act_logits if (last and commit_delta) else None,
                             self.delta if (last and commit_delta) else None, self.ws, self.ws_bytes)
            B.polestar_refresh(self.h, Ls, blk_start, self.h_act[cur_h], sel, None, None, None,
                               self.h_act[1 - cur_h], self.pk_rows[pk], self.ws, self.ws_bytes)
            u_in = sel if refresh else None
            cur_h = 1 - cur_h
            pk = 1 - pk
        self.last_packet = 1 - pk
        return self.h_act[cur_h]
