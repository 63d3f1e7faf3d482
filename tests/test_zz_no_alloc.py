"""polestar_step_noalloc (the refresh step with the library's static scratch as workspace)
against polestar_step with a caller workspace: bit-identical outputs and state, on two calls
in a row, the second with a smaller stack (fewer layers, one sequence, fewer positions), so
that it runs on the scratch contents the first call left behind."""
from __future__ import annotations

import pytest
import torch

import synth
from drift_driven_sparse_amd import binding as B
from drift_driven_sparse_amd.stack import RefreshStack
from tests.harness import log
from tests.test_gpu_stack import _outputs, _restore, _snapshot

pytestmark = pytest.mark.gpu


def _stack(w, batch, n_layers):
    dims = B.Dims(d=w.d, n_heads=w.n_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ffn=w.ffn,
                  n_pos=w.n_pos, batch=batch, block=w.block, win_prefix=w.win_prefix, win_suffix=w.win_suffix,
                  n_clusters=w.n_clusters, top_k=w.top_k, vocab=0, dtype=B.BF16, resid_fmt=B.RESID_RAW)
    params = B.Params(rms_eps=w.rms_eps, tau_s=w.tau_s, tau_suf=w.tau_suf, alpha=w.alpha, hist=w.hist, mask_id=0,
                      kmeans_iters=w.kmeans_iters)
    st = RefreshStack(dims, params, n_layers)
    nw = w.win_prefix + w.win_suffix
    for l in range(n_layers):
        st.set_layer_weights(l, synth.layer_weights(w, l, device="cuda"))
    h0 = torch.stack([synth.embeddings(w, 0, "cuda", b).to(torch.bfloat16) for b in range(batch)]).contiguous()
    inits = [torch.stack([torch.tensor(synth.kmeans_init(w, nw, l, 0, 0, b), dtype=torch.int32)
                          for b in range(batch)]).cuda() for l in range(n_layers)]
    st.entry_forward(w.prompt, h0, inits, full=True)
    torch.cuda.synchronize()
    return st


def test_step_noalloc_matches_step():
    cases = [("tiny bf16, 3 layers, batch 2, n 320", synth.shrink(synth.WORKLOADS[1], dtype="bf16"), 2, 3),
             ("tiny bf16, 2 layers, batch 1, n 128", synth.shrink(synth.WORKLOADS[1], dtype="bf16", gen=64), 1, 2)]
    for name, w, batch, n_layers in cases:
        st = _stack(w, batch, n_layers)
        try:
            assert st.ws_bytes <= B.SCRATCH_BYTES
            snap = _snapshot(st)
            x = synth.tensor(w, (97,), (batch, w.block, w.d), 1.0, 0, "cuda", "bf16")
            layers = [st.struct(l) for l in range(n_layers)]
            results = []
            for noalloc in (False, True):
                _restore(st, snap)
                for L in st.layers:                    # the query caches start from the entry's state
                    L["q_ok"].zero_()
                st.h_act[0].copy_(x)
                for pk in st.pk_cnt:
                    pk.zero_()
                args = (st.h, B.DRIFT_REFRESH, layers, w.prompt, st.h_act[0], st.h_act[1], st.packets[0],
                        st.packets[1], st.D, st.topk, st.act_logits, st.delta)
                if noalloc:
                    B.polestar_step_noalloc(*args)
                else:
                    B.polestar_step(*args, st.ws, st.ws_bytes)
                torch.cuda.synchronize()
                results.append(_outputs(st, st.h_act[n_layers % 2]))
            want, got = results
            bad = [k for k in want if not torch.equal(got[k], want[k])]
            log(f"[no-alloc] {name}: {len(want) - len(bad)}/{len(want)} tensors bit-identical")
            assert not bad, f"{name}: polestar_step_noalloc differs from polestar_step in {bad}"
        finally:
            st.close()
