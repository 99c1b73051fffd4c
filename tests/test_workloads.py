"""The seeded synthetic inputs reproduce their recipes (CPU only)."""
import numpy as np
import torch

import workloads as w


def test_expert_counts_and_offsets():
    for name, cfg in w.MLP_CONFIGS.items():
        counts = w.expert_counts(name)
        assert counts == w.KNOWN_COUNTS[name]
        offs = w.padded_offsets(counts, cfg["pad"])
        assert all(o % cfg["pad"] == 0 for o in offs)
        assert all(offs[e + 1] - offs[e] >= counts[e] for e in range(len(counts)))
    assert sum(w.expert_counts("dsv3_rank")) == 24576
    assert w.padded_offsets(w.expert_counts("dsv3_rank"), 256)[-1] == 26112
    assert w.padded_offsets(w.expert_counts("large_expert"), 256)[-1] == 33792
    assert w.padded_offsets(w.expert_counts("tiny"), 128)[-1] == 1280


def test_tiny_problem_layout():
    p = w.mlp_problem("tiny", m_capacity=1536, pad_fill=float("nan"), tail_fill=float("nan"))
    x, offs, counts = p["x"], p["offs"], p["counts"]
    assert x.shape == (1536, 256) and x.dtype == torch.bfloat16
    # every token row appears in exactly topk=2 experts
    choice = w.tiny_routing()
    rows = torch.cat([x[offs[e]:offs[e] + counts[e]] for e in range(4)])
    assert rows.shape[0] == 2 * choice.shape[0]
    assert torch.isnan(x[offs[0] + counts[0]:offs[1]]).all() and torch.isnan(x[1280:]).all()
    assert not torch.isnan(rows).any()
    assert abs(float(rows.float().std()) - 1.0) < 0.05
    assert abs(float(p["w1"].float().std()) - 0.02) < 0.002


def test_quant_matrix_recipe():
    a = w.quant_matrix(4096, 2048, seed=3)
    assert a.dtype == torch.bfloat16 and a.shape == (4096, 2048)
    blocks = a.float().view(4096, 64, 32).abs().amax(-1)
    zero = (blocks == 0).float().mean().item()
    big = (blocks > 1000).float().mean().item()
    small = ((blocks > 0) & (blocks < 1e-3)).float().mean().item()
    assert 0.0005 < zero < 0.01 and 0.002 < big < 0.01 and 0.002 < small < 0.01
    b = w.quant_matrix(4096, 2048, seed=3)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    cols = a.float().view(128, 32, 2048).abs().amax(1)
    assert (cols == 0).any()
