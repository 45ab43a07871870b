"""The seeded input generators produce the shapes the workloads call for (CPU)."""

import numpy as np
import torch

import workloads as W


def depth(parent, i):
    d = 0
    while i != -1:
        i = parent[i]
        d += 1
    return d


def test_top8_tree_is_width8_depth8():
    parent, scores = W.top8_tree(np.random.default_rng(1))
    assert len(parent) == 64
    assert all(p == -1 or 0 <= p < i for i, p in enumerate(parent))
    assert sum(p == -1 for p in parent) == 8
    for r in range(8):
        for i in range(8 * r, 8 * r + 8):
            assert depth(parent, i) == r + 1
            if r:
                assert 8 * (r - 1) <= parent[i] < 8 * r
    # scores are path log-likelihoods: a child never scores above its parent
    assert all(p == -1 or scores[i] <= scores[p] for i, p in enumerate(parent))


def test_generators_are_deterministic_per_seed():
    a = W.make_inputs(W.config("llama3_8b_verify"))
    b = W.make_inputs(W.config("llama3_8b_verify"))
    assert a["parent"] == b["parent"]
    assert torch.equal(a["q"], b["q"])
    assert torch.equal(a["k"][..., :2048 + 64, :], b["k"][..., :2048 + 64, :])


def test_inputs_are_poisoned_beyond_the_tree():
    cfg = W.config("tiny_fp32")
    x = W.make_inputs(cfg)
    end = cfg["prefix"] + cfg["n_tree"]
    assert torch.isnan(x["k"][..., end:, :]).all() and torch.isfinite(x["k"][..., :end, :]).all()
    assert x["q"].dtype == torch.float32 and x["q"].shape == (15, 2, 64)


def test_bf16_inputs_are_rounded_float32_draws():
    cfg = W.config("llama3_8b_verify")
    x = W.make_inputs(cfg)
    assert x["q"].dtype == torch.bfloat16
    rng = np.random.default_rng(cfg["seed"])
    W.make_tree(cfg, rng)
    raw = rng.standard_normal(size=(64, 32, 128), dtype=np.float32) * np.float32(cfg["value_scale"])
    assert torch.equal(torch.from_numpy(raw).to(torch.bfloat16), x["q"])


def test_descendants_and_paths():
    parent = [-1, 0, 0, 1, 1, 2, 3, -1]
    assert W.descendants(parent, 1) == [3, 4, 6]
    assert W.descendants(parent, -1) == list(range(8))
    rng = np.random.default_rng(3)
    for _ in range(50):
        path = W.draft_path(rng, parent)
        assert parent[path[0]] == -1
        assert all(parent[b] == a for a, b in zip(path, path[1:]))


def test_refill_grows_back_to_64_and_restarts_when_empty():
    rng = np.random.default_rng(4)
    parent, scores = W.refill(rng, [-1, 0, 0], [-0.1, -0.5, -0.7], 64)
    assert len(parent) == 64 and parent[:3] == [-1, 0, 0]
    assert all(p == -1 or 0 <= p < i for i, p in enumerate(parent))
    parent, _ = W.refill(rng, [], [], 64)
    assert len(parent) == 64 and sum(p == -1 for p in parent) == 8


def test_draft_loop_state_machine():
    cfg = W.config("draft_loop_1b")
    loop = W.DraftLoop(cfg)
    for _ in range(20):
        path, surv = loop.choose()
        assert 1 <= len(path) <= 8
        new_parent = [-1 if loop.parent[s] == path[-1] else surv.index(loop.parent[s]) for s in surv]
        keep, kr, vr = loop.advance(surv, new_parent, loop.prefix_len + len(path))
        assert keep == len(surv) and len(loop.parent) == 64
        assert kr.shape == (1, 8, 64 - keep, 64)


def test_mask_probe_layout():
    cfg = W.config("llama3_8b_verify")
    x = W.mask_probe_inputs(cfg, [-1, 0, 1])
    assert x["q"][..., 0].eq(16).all() and x["k"][0, :, :2048, 0].eq(-16).all()
    assert x["v"][0, 3, 2048 + 2, 2] == 1
