"""Seeded input generator: determinism, shapes, recipe (CPU only)."""

import numpy as np
import torch

from gated_delta_rule_04_amd import inputs


def test_deterministic_and_blocked_draws_match_one_draw(monkeypatch):
    a = inputs.make_prefill(2, 33, 3, 64, 32, "bf16", 1, seed=5)
    monkeypatch.setattr(inputs, "_BLOCK_ELEMS", 100)   # force many small blocks
    b = inputs.make_prefill(2, 33, 3, 64, 32, "bf16", 1, seed=5)
    for key in ("q", "k", "v", "g", "beta"):
        assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16)), key


def test_recipe_properties():
    d = inputs.make_prefill(1, 4096, 2, 64, 64, "f32", 1, seed=1)
    qn = d["q"].double().norm(dim=-1)
    assert torch.allclose(qn, torch.ones_like(qn), atol=1e-6)
    assert float(d["g"].max()) <= 0.0
    assert 0.0 < float(d["beta"].min()) and float(d["beta"].max()) < 1.0
    alpha = d["g"].double().exp()
    assert abs(float(alpha.mean()) - 0.845) < 0.01   # E[sigmoid(2 - z)], z ~ N(0,1)


def test_bf16_is_rne_of_f32():
    d32 = inputs.make_prefill(1, 16, 1, 64, 64, "f32", 1, seed=3)
    d16 = inputs.make_prefill(1, 16, 1, 64, 64, "bf16", 1, seed=3)
    assert torch.equal(d32["v"].to(torch.bfloat16).view(torch.int16), d16["v"].view(torch.int16))


def test_doc_lengths():
    lens = inputs.doc_lengths(65536, 2003)
    assert sum(lens) == 65536
    assert min(lens) >= 16 and max(lens) <= 8192
    assert 20 <= len(lens) <= 100
    assert lens == inputs.doc_lengths(65536, 2003)


def test_g64_shape_and_decode_shapes():
    d = inputs.make_prefill(1, 8, 2, 128, 128, "bf16", 64, seed=0)
    assert tuple(d["g"].shape) == (1, 8, 2, 2)
    r = inputs.make_decode(2, 3, 64, 64, steps=2, seed=0)
    assert tuple(r["state"].shape) == (2, 3, 64, 64) and r["state"].dtype == torch.float32
    assert abs(float(r["state"].std()) - 0.02) < 0.002
    assert tuple(r["steps"][1]["beta"].shape) == (2, 3)
    # fewer steps give the same first steps (per-step draws come in step order)
    r1 = inputs.make_decode(2, 3, 64, 64, steps=1, seed=0)
    assert torch.equal(r1["steps"][0]["q"].view(torch.int16), r["steps"][0]["q"].view(torch.int16))
