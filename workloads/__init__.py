"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module draws random numbers and builds tree shapes. It contains none of
the arithmetic of tree attention or of the re-root (that lives separately in the
oracle and in the HIP library), so both sides can be fed the same inputs.

Workload shapes follow the SwiftSpec pages (arXiv 2506.11309, Pith review
page): the verify tree of the pages' operating point is expanded with width 8
by maximum likelihood, i.e. by the sum of log-softmax scores along each path
("Assumptions & free parameters": draft expansion width and the
maximum-likelihood expansion assumption). Verified-path lengths of 1..8 stand
in for the pages' target batch of 8 tokens. The pages' own datasets and models
are not available; these seeded Gaussian inputs stand in for them.

Values are drawn in float32 with ``numpy.random.default_rng(seed)`` (PCG64) and
rounded to bfloat16 (round-to-nearest-even, via torch) for bf16 workloads.
"""

import math

import numpy as np
import torch

# name -> shape/seed recipe. capacity defaults to prefix + 256.
CONFIGS = {
    "tiny_fp32": dict(n_q_heads=2, n_kv_heads=1, head_dim=64, dtype="f32", prefix=128,
                      n_tree=15, capacity=256, seed=0, value_scale=1.0, tree="random", vocab=1000, layers=2),
    "llama3_8b_verify": dict(n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
                             prefix=2048, n_tree=64, capacity=2048 + 256, seed=1,
                             value_scale=1.0 / math.sqrt(128), tree="top8", vocab=128256, layers=32),
    "llama3_70b_verify": dict(n_q_heads=64, n_kv_heads=8, head_dim=128, dtype="bf16",
                              prefix=8192, n_tree=64, capacity=8192 + 256, seed=2,
                              value_scale=1.0 / math.sqrt(128), tree="top8", vocab=128256, layers=80),
    "qwen2_72b_32k_verify": dict(n_q_heads=64, n_kv_heads=8, head_dim=128, dtype="bf16",
                                 prefix=32768, n_tree=64, capacity=32768 + 256, seed=3,
                                 value_scale=1.0 / math.sqrt(128), tree="top8", vocab=152064, layers=80),
    "draft_loop_1b": dict(n_q_heads=32, n_kv_heads=8, head_dim=64, dtype="bf16",
                          prefix=4096, n_tree=64, capacity=8192, seed=4,
                          value_scale=1.0 / 8.0, tree="top8", iterations=100, vocab=128256, layers=16),
    # The pages' operating point: a verify tree of bs = 8 nodes at 70B shapes
    # (the 8 most likely nodes of the width-8 expansion; HBM-bound).
    "llama3_70b_verify_bs8": dict(n_q_heads=64, n_kv_heads=8, head_dim=128, dtype="bf16",
                                  prefix=8192, n_tree=8, capacity=8192 + 256, seed=5,
                                  value_scale=1.0 / math.sqrt(128), tree="top8_bs8", vocab=128256, layers=80),
    # One tensor-parallel rank's share of the 70B verify step when the target
    # runs attention on 4 GPUs split by KV head (16 query / 2 KV heads).
    "llama3_70b_verify_tp4": dict(n_q_heads=16, n_kv_heads=2, head_dim=128, dtype="bf16",
                                  prefix=8192, n_tree=64, capacity=8192 + 256, seed=7,
                                  value_scale=1.0 / math.sqrt(128), tree="top8", vocab=128256, layers=80),
    # A draft-expansion step: only the w = 8 newest leaves of the 64-node tree
    # are queries, against the whole [prefix | tree].
    "draft_expand_w8": dict(n_q_heads=32, n_kv_heads=8, head_dim=64, dtype="bf16",
                            prefix=4096, n_tree=64, q_first=56, capacity=4096 + 256, seed=6,
                            value_scale=1.0 / 8.0, tree="top8", vocab=128256, layers=16),
}

# vocab: the model family's vocabulary (Llama 3: 128256 token ids, Qwen2:
# 152064), the row length of the target's logits in tree verification.
# layers: the model's decoder layers (Llama 3 8B: 32, 70B: 80, Qwen2-72B: 80,
# the Llama 3.2 1B draft: 16), i.e. the depth of the cache that one re-root
# call moves.

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def config(name, **overrides):
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


# ----------------------------------------------------------------------------- trees

def random_parent(rng, n):
    """``parent[0] = -1`` and ``parent[i]`` uniform in ``0..i-1`` (a single-root tree)."""
    return [-1] + [int(rng.integers(0, i)) for i in range(1, n)]


def _log_softmax(z):
    z = np.asarray(z, dtype=np.float64)
    m = z.max()
    return z - (m + math.log(np.exp(z - m).sum()))


def _expand(rng, frontier, scores, width, keep):
    """One maximum-likelihood expansion round.

    Every frontier node proposes ``width`` children scored by its own score plus
    the log-softmax of fresh N(0,1) logits; the best ``keep`` candidates survive,
    returned in (parent position in frontier, slot) order. Ties have
    probability zero and are broken by that order.
    """
    cands = []
    for pos, node in enumerate(frontier):
        base = 0.0 if node < 0 else scores[node]
        ls = _log_softmax(rng.standard_normal(width))
        for slot in range(width):
            cands.append((base + ls[slot], pos, slot, node))
    best = sorted(range(len(cands)), key=lambda c: (-cands[c][0], c))[:keep]
    best.sort()
    return [(cands[c][3], cands[c][0]) for c in best]


def top8_tree(rng, width=8, rounds=8):
    """Width-8 maximum-likelihood tree: ``(parent, scores)`` with ``width*rounds`` nodes.

    Round 0 puts ``width`` children under the virtual root. Each later round lets
    every node of the previous round propose ``width`` children and keeps the
    global top ``width``. Nodes are numbered in round order, so ``parent[i] < i``.
    """
    parent, scores = [], []
    frontier = [-1]
    for _ in range(rounds):
        kept = _expand(rng, frontier, scores, width, width)
        frontier = []
        for par, sc in kept:
            frontier.append(len(parent))
            parent.append(par)
            scores.append(sc)
    return parent, scores


def children(parent):
    kids = [[] for _ in parent]
    for i, p in enumerate(parent):
        if p >= 0:
            kids[p].append(i)
    return kids


def descendants(parent, node):
    """Strict descendants of ``node`` in ascending order (``node = -1``: every node)."""
    if node < 0:
        return list(range(len(parent)))
    inside = {node}
    out = []
    for i in range(node + 1, len(parent)):
        if parent[i] in inside:
            inside.add(i)
            out.append(i)
    return out


def random_path_from(rng, parent, start, max_len=None):
    """Walk from ``start`` down uniformly random children until a leaf or ``max_len``."""
    kids = children(parent)
    path = [start]
    while kids[path[-1]] and (max_len is None or len(path) < max_len):
        path.append(int(kids[path[-1]][rng.integers(0, len(kids[path[-1]]))]))
    return path


def draft_path(rng, parent, max_len=8):
    """Accepted path of the draft loop: length L ~ U{1..max_len}, started at a
    uniformly chosen first-level node and walked down random children."""
    want = int(rng.integers(1, max_len + 1))
    roots = [i for i, p in enumerate(parent) if p == -1]
    return random_path_from(rng, parent, int(roots[rng.integers(0, len(roots))]), want)


def refill(rng, parent, scores, n_target=64, width=8):
    """Grow a re-rooted tree back to ``n_target`` nodes by maximum-likelihood rounds.

    Each round every current leaf proposes ``width`` children; the best
    ``min(width, room)`` are appended. An empty tree restarts from the virtual
    root. Returns the new ``(parent, scores)``; appended nodes get indices after
    the existing ones, so ``parent[i] < i`` still holds.
    """
    parent, scores = list(parent), list(scores)
    while len(parent) < n_target:
        room = n_target - len(parent)
        if not parent:
            frontier = [-1]
        else:
            kids = children(parent)
            frontier = [i for i in range(len(parent)) if not kids[i]]
        for par, sc in _expand(rng, frontier, scores, width, min(width, room)):
            parent.append(par)
            scores.append(sc)
    return parent, scores


def best_nodes(parent, scores, k):
    """The ``k`` highest-scoring nodes (ties: lower index first), renumbered in
    ascending order. Scores are sums of log-probabilities along the path, so a
    child never outscores its parent and the kept set is closed under parents."""
    keep = sorted(sorted(range(len(parent)), key=lambda i: (-scores[i], i))[:k])
    new = {old: j for j, old in enumerate(keep)}
    return [new[parent[i]] if parent[i] >= 0 else -1 for i in keep], [scores[i] for i in keep]


def make_tree(cfg, rng):
    if cfg["tree"] == "random":
        return random_parent(rng, cfg["n_tree"]), None
    parent, scores = top8_tree(rng)
    if cfg["tree"] == "top8_bs8":
        parent, scores = best_nodes(parent, scores, cfg["n_tree"])
    assert len(parent) == cfg["n_tree"]
    return parent, scores


# ----------------------------------------------------------------------------- tensors

def _draw(rng, shape, scale, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return torch.from_numpy(x).to(TORCH_DTYPE[dtype])


def make_inputs(cfg, rng=None, n_layers=1, poison=True, value_scale=None):
    """Seeded q and KV cache for one config; all CPU torch tensors.

    Returns a dict with ``q [n_tree - q_first, n_q_heads, head_dim]`` (the
    query rows are the tree nodes from ``cfg["q_first"]``, default 0) and
    ``k, v [n_layers, n_kv_heads, capacity, head_dim]``, ``parent``, ``scores``,
    ``prefix_len``. Slots at or beyond ``prefix + n_tree`` are NaN when
    ``poison`` (they must never be read), random otherwise.
    """
    if rng is None:
        rng = np.random.default_rng(cfg["seed"])
    scale = cfg["value_scale"] if value_scale is None else value_scale
    parent, scores = make_tree(cfg, rng)
    n, hq, hkv, d = cfg["n_tree"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    cap = cfg["capacity"]
    q = _draw(rng, (n - cfg.get("q_first", 0), hq, d), scale, cfg["dtype"])
    k = _draw(rng, (n_layers, hkv, cap, d), scale, cfg["dtype"])
    v = _draw(rng, (n_layers, hkv, cap, d), scale, cfg["dtype"])
    if poison:
        end = cfg["prefix"] + n
        k[:, :, end:] = float("nan")
        v[:, :, end:] = float("nan")
    return dict(q=q, k=k, v=v, parent=parent, scores=scores, prefix_len=cfg["prefix"], q_first=cfg.get("q_first", 0))


def mask_probe_inputs(cfg, parent, n_layers=1):
    """Inputs whose output spells out the mask.

    Every query is ``16 e_0`` and every prefix key ``-16 e_0``, so prefix weights
    are negligible (score ``-256/sqrt(head_dim)``), tree keys are zero (equal
    scores), and tree value row ``j`` is the unit vector ``e_j``. The exact output
    of node ``i`` is then ``1/|A|`` on the coordinates of its visible tree set
    ``A`` and (almost) 0 elsewhere. Requires ``n_tree <= head_dim``.
    """
    n, hq, hkv, d = len(parent), cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    assert n <= d
    P, cap = cfg["prefix"], cfg["capacity"]
    dt = TORCH_DTYPE[cfg["dtype"]]
    q = torch.zeros((n, hq, d), dtype=dt)
    q[:, :, 0] = 16.0
    k = torch.zeros((n_layers, hkv, cap, d), dtype=dt)
    v = torch.zeros((n_layers, hkv, cap, d), dtype=dt)
    k[:, :, :P, 0] = -16.0
    for j in range(n):
        v[:, :, P + j, j] = 1.0
    k[:, :, P + n:] = float("nan")
    v[:, :, P + n:] = float("nan")
    return dict(q=q, k=k, v=v, parent=list(parent), scores=None, prefix_len=P)


def to_f64(t):
    """Exact float64 copy of a float32/bfloat16 tensor, as numpy."""
    return t.detach().to("cpu", torch.float64).numpy()


def bits_to_f64(bits):
    """float64 values of stored words (uint16 = bf16, uint32 = fp32); exact."""
    bits = np.asarray(bits)
    if bits.dtype == np.uint16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float32).astype(np.float64)


def raw_bits(t):
    """The stored words of a cache tensor (uint16 for bf16, uint32 for fp32)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


class DraftLoop:
    """Seeded driver of the draft-loop workload (state = tree + prefix length).

    Each iteration: fresh queries for all tree nodes, an accepted path of length
    1..8 from a first-level node, the surviving subtree (every descendant of the
    last accepted node), then a refill back to 64 nodes whose new cache rows get
    fresh random K/V.
    """

    def __init__(self, cfg, seed=None):
        self.cfg = cfg
        self.rng = np.random.default_rng(cfg["seed"] if seed is None else seed)
        self.prefix_len = cfg["prefix"]
        self.parent, self.scores = top8_tree(self.rng)

    def initial_cache(self, n_layers=1):
        c = self.cfg
        shape = (n_layers, c["n_kv_heads"], c["capacity"], c["head_dim"])
        k = _draw(self.rng, shape, c["value_scale"], c["dtype"])
        v = _draw(self.rng, shape, c["value_scale"], c["dtype"])
        return k, v

    def queries(self):
        c = self.cfg
        return _draw(self.rng, (len(self.parent), c["n_q_heads"], c["head_dim"]),
                     c["value_scale"], c["dtype"])

    def choose(self):
        path = draft_path(self.rng, self.parent)
        return path, descendants(self.parent, path[-1])

    def advance(self, survivors, new_parent, new_prefix_len, n_layers=1):
        """Adopt the re-rooted tree and refill it.

        Returns ``(first_new_node, k_rows, v_rows)``: the K/V rows to write at
        slots ``new_prefix_len + first_new_node ..`` of every layer.
        """
        c = self.cfg
        scores = [self.scores[s] for s in survivors]
        keep = len(new_parent)
        self.parent, self.scores = refill(self.rng, new_parent, scores, c["n_tree"])
        self.prefix_len = new_prefix_len
        add = len(self.parent) - keep
        shape = (n_layers, c["n_kv_heads"], add, c["head_dim"])
        return keep, _draw(self.rng, shape, c["value_scale"], c["dtype"]), \
            _draw(self.rng, shape, c["value_scale"], c["dtype"])


def make_verify_inputs(cfg, parent, rng=None, accept=0.8, logit_scale=2.0):
    """Target logits and drafted tokens for verifying the tree ``parent``.

    Rows (root, then one per node) are N(0, 1) * ``logit_scale`` with one
    planted maximum per row (its row maximum + 1, at a uniform token id);
    below each row's owner (the virtual root, or node ``j`` for row ``1 + j``)
    one uniformly chosen child drafts the planted token with probability
    ``accept``, every other child drafts a different uniform token. So the
    accepted depth follows ``accept`` the way a draft model's agreement with
    the target would. Returns ``logits`` (torch, cfg dtype, CPU) and
    ``tokens`` (torch int32, CPU).
    """
    rng = np.random.default_rng(cfg["seed"] + 1000) if rng is None else rng
    n, vocab = len(parent), cfg["vocab"]
    x = rng.standard_normal((n + 1, vocab), dtype=np.float32) * np.float32(logit_scale)
    planted = rng.integers(0, vocab, size=n + 1)
    x[np.arange(n + 1), planted] = x.max(axis=1) + np.float32(1.0)
    kids = children(parent)
    roots = [i for i in range(n) if parent[i] < 0]
    tokens = np.empty(n, dtype=np.int32)
    for owner in [-1] + list(range(n)):
        c = roots if owner < 0 else kids[owner]
        if not c:
            continue
        want = int(planted[owner + 1])
        hit = int(rng.integers(0, len(c))) if rng.random() < accept else -1
        for k, node in enumerate(c):
            t = int(rng.integers(0, max(vocab - 1, 1)))
            tokens[node] = want if k == hit else (t if t < want else t + 1)
    return dict(logits=torch.from_numpy(x).to(TORCH_DTYPE[cfg["dtype"]]), tokens=torch.from_numpy(tokens))


def make_expand_inputs(cfg, w, rng=None, logit_scale=2.0):
    """Draft logits and path scores of a frontier of ``w`` leaves.

    Logits are N(0, 1) * ``logit_scale`` over the model's vocabulary (cfg
    dtype); path scores are float32 sums of 1..8 draws of -Exp(1) (a leaf
    at depth d has d log-probabilities along its path). Returns ``logits``
    (torch, CPU) and ``path_scores`` (torch float32, CPU).
    """
    rng = np.random.default_rng(cfg["seed"] + 2000) if rng is None else rng
    x = rng.standard_normal((w, cfg["vocab"]), dtype=np.float32) * np.float32(logit_scale)
    depth = rng.integers(1, 9, size=w)
    s = np.array([-rng.exponential(1.0, size=d).sum() for d in depth], dtype=np.float32)
    return dict(logits=torch.from_numpy(x).to(TORCH_DTYPE[cfg["dtype"]]), path_scores=torch.from_numpy(s))
