"""The page's printed defaults and sweep ranges (tests/golden/table5_defaults.json, copied from
the page's §5.1 and Table 5) against the synthetic workloads and the parity cases: the
workloads use the defaults, and every swept value a parity case uses lies in the page's range
(block size 8 aside: the page's short-generation benchmark setting, outside Table 5)."""
import json
import os

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "table5_defaults.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_workloads_use_the_page_defaults():
    g = _golden()["defaults"]
    for w in synth.WORKLOADS.values():
        assert w.block == g["block"]
        assert (w.win_prefix, w.win_suffix) == (g["win_prefix_blocks"] * w.block, g["win_suffix_blocks"] * w.block)
        assert (w.n_clusters, w.top_k, w.tau_upd, w.hist) == (g["n_clusters"], g["top_k"], g["tau_upd"], g["hist"])
        assert (w.tau_s, w.alpha, w.tau_suf) == (g["tau_s"], g["alpha"], g["tau_suf"])
    assert synth.WORKLOADS[5].resid == g["resid"]


def test_parity_sweeps_stay_in_the_page_ranges():
    from tests import test_gpu_commit, test_gpu_layer_parity
    sw = _golden()["sweeps"]
    for name, (w, _, _) in test_gpu_layer_parity.CASES.items():
        if not name.startswith("sweep_"):
            continue
        assert w.block in sw["block"] + [8], name
        assert w.n_clusters in sw["n_clusters"], name
        assert w.top_k in sw["top_k_at_K8"], name
        assert w.win_prefix % w.block == 0 and w.win_suffix % w.block == 0, name
        assert [w.win_prefix // w.block, w.win_suffix // w.block] in sw["window_blocks"], name
    for name, (w, _, _) in test_gpu_commit.CASES.items():
        assert w.hist in sw["hist"], name
        assert w.alpha in sw["alpha"], name
