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


def test_verify_inputs_plant_one_maximum_per_row_and_follow_accept():
    cfg = W.config("llama3_8b_verify", vocab=3000)
    parent, _ = W.make_tree(cfg, np.random.default_rng(cfg["seed"]))
    for accept, seed in ((1.0, 1), (0.0, 2)):
        x = W.make_verify_inputs(cfg, parent, np.random.default_rng(seed), accept=accept)
        logits = W.to_f64(x["logits"])
        assert logits.shape == (len(parent) + 1, 3000) and x["tokens"].dtype == torch.int32
        top = np.sort(logits, axis=1)
        assert (top[:, -1] > top[:, -2]).all()  # a unique maximum, even after bf16 rounding
        choice = logits.argmax(axis=1)
        kids = W.children(parent)
        for owner in [-1] + list(range(len(parent))):
            c = [i for i in range(len(parent)) if parent[i] == owner] if owner < 0 else kids[owner]
            hits = sum(int(x["tokens"][i]) == choice[owner + 1] for i in c)
            assert hits == ((1 if c else 0) if accept == 1.0 else 0)


def test_expand_inputs_are_seeded_and_shaped():
    cfg = W.config("draft_expand_w8")
    a = W.make_expand_inputs(cfg, 8, np.random.default_rng(3))
    b = W.make_expand_inputs(cfg, 8, np.random.default_rng(3))
    assert torch.equal(a["logits"], b["logits"]) and torch.equal(a["path_scores"], b["path_scores"])
    assert a["logits"].shape == (8, 128256) and a["logits"].dtype == torch.bfloat16
    assert a["path_scores"].dtype == torch.float32 and (a["path_scores"] < 0).all()
