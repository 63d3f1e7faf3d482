"""The seeded input generator: determinism, distribution and the workload recipes."""
import math

import numpy as np
import torch

import synth


def test_hash32_matches_scalar_reference():
    xs = [0, 1, 2, 0xDEADBEEF, 0xFFFFFFFF, 123456789]
    t = synth.hash32(torch.tensor(xs, dtype=torch.int64)).tolist()
    assert t == [synth.hash32_int(x) for x in xs]
    assert synth.hash32_int(1) != synth.hash32_int(2)


def test_normal_is_deterministic_and_standard():
    a = synth.normal((1000, 300), 1.0, 99)
    b = synth.normal((1000, 300), 1.0, 99)
    assert torch.equal(a, b)
    assert not torch.equal(a, synth.normal((1000, 300), 1.0, 100))
    v = a.double()
    assert abs(v.mean().item()) < 0.01 and abs(v.std().item() - 1.0) < 0.01
    # a quarter of the mass lies beyond the 75% quantile
    assert abs((v > 0.6744897501960817).double().mean().item() - 0.25) < 0.01


def test_bf16_weights_are_rounded_fp32_draws():
    w = synth.WORKLOADS[1]
    f32 = synth.weight(w, 0, "wq", dtype="f32")
    b16 = synth.weight(w, 0, "wq", dtype="bf16")
    assert torch.equal(f32.to(torch.bfloat16), b16)
    assert abs(f32.double().std().item() - 1 / math.sqrt(w.d)) < 0.02 / math.sqrt(w.d)


def test_unmask_schedule_covers_blocks():
    w = synth.shrink(synth.WORKLOADS[1], steps=200)
    sch = synth.unmask_schedule(w, 0)
    per_block = {}
    for b, offs in sch:
        assert 1 <= len(offs) <= 4
        per_block.setdefault(b, []).extend(offs)
    for b, offs in per_block.items():
        assert len(offs) == len(set(offs))
    assert sorted(per_block[0]) == list(range(32))


def test_workload_shapes():
    W = synth.WORKLOADS
    assert W[3].n_pos == 1024 and W[3].n_layers == 32 and W[3].d == 4096
    assert W[4].n_heads == 28 and W[4].n_kv_heads == 4 and W[4].ffn == 18944
    assert W[5].batch == 16 and W[5].resid == "nvfp4" and W[5].vocab == 126464
