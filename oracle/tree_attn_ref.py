"""Tree-masked attention, written out as its definition in float64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
may import this module.

Source: SwiftSpec (arXiv 2506.11309), Pith review page. "What carries the
argument" and "Core claim" fix the cache layout: verified tokens form a
contiguous prefix and the draft-tree tokens follow it. The referee summary says
the target consumes tree-structured inputs through masked attention. What a
tree token may see is left implicit. The plain reading, used here: the whole
prefix, every ancestor in the tree, and itself.

Two formulations are kept on purpose. They are written independently so that
each can check the other:

* ``tree_attn_ref`` walks the parent links of each node and gathers that
  node's key set explicitly, one (node, head) at a time;
* ``tree_attn_dense_ref`` builds the full boolean visibility matrix by
  transitive closure (repeated boolean matrix products) and applies a dense
  masked softmax with ``-inf``.
"""

import math

import numpy as np


def check_parent(parent):
    """Validate a parent array: ``parent[i]`` is -1 or an earlier node index.

    Returns the array as a list of Python ints. Raises ``ValueError`` otherwise.
    """
    par = [int(p) for p in parent]
    for i, p in enumerate(par):
        if not (p == -1 or 0 <= p < i):
            raise ValueError(f"parent[{i}] = {p} is neither -1 nor in [0, {i})")
    return par


def ancestors_inclusive(parent, i):
    """Node ``i`` together with every node met on the walk up to the virtual root.

    The walk follows ``parent`` links until it reaches -1 (the last verified
    token, which already sits in the prefix). Returned in ascending order.
    """
    seen = []
    j = int(i)
    while j != -1:
        seen.append(j)
        j = int(parent[j])
    return sorted(seen)


def visibility_matrix(parent):
    """Boolean ``[n, n]`` matrix: entry ``(i, j)`` is True iff tree token ``j``
    is ``i`` itself or an ancestor of ``i``.

    Built as the reflexive-transitive closure of the child-to-parent relation,
    by squaring the boolean reachability matrix until it stops changing. This
    route shares nothing with the parent walk in ``ancestors_inclusive``.
    """
    par = check_parent(parent)
    n = len(par)
    reach = np.eye(n, dtype=bool)
    for i, p in enumerate(par):
        if p >= 0:
            reach[i, p] = True
    while True:
        nxt = (reach.astype(np.int64) @ reach.astype(np.int64)) > 0
        if np.array_equal(nxt, reach):
            return reach
        reach = nxt


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k_layer, v_layer, prefix_len, n_tree, n_kv_heads, q_first=0):
    if q.ndim != 3 or k_layer.ndim != 3 or v_layer.shape != k_layer.shape:
        raise ValueError("q must be [n_rows, n_q_heads, head_dim]; k, v [n_kv_heads, capacity, head_dim]")
    n, hq, d = q.shape
    if not 0 <= q_first <= n_tree:
        raise ValueError("q_first must be in [0, n_tree]")
    if n != n_tree - q_first:
        raise ValueError("q rows must equal the number of tree nodes from q_first on")
    if k_layer.shape[0] != n_kv_heads or k_layer.shape[2] != d:
        raise ValueError("k/v head count or head_dim mismatch")
    if hq % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if prefix_len < 0 or prefix_len + n_tree > k_layer.shape[1]:
        raise ValueError("prefix_len + n_tree exceeds the cache capacity")


def tree_attn_ref(q, k_layer, v_layer, prefix_len, parent, n_kv_heads, q_first=0):
    """Tree-masked attention of every (node, query head), one at a time.

    Arguments:
        q: ``[n_tree - q_first, n_q_heads, head_dim]``: row ``r`` is the query
            of tree node ``q_first + r``.
        k_layer, v_layer: ``[n_kv_heads, capacity, head_dim]``: one layer of the
            cache. Slot ``t < prefix_len`` holds verified token ``t``; slot
            ``prefix_len + j`` holds tree node ``j``. Slots at or beyond
            ``prefix_len + n_tree`` are never read.
        prefix_len: number of verified tokens.
        parent: ``parent[i]`` in ``{-1} U [0, i)``.
        n_kv_heads: KV heads; query head ``h`` uses KV head
            ``h // (n_q_heads // n_kv_heads)``.
        q_first: the first tree node that has a query (0: all of them). The
            draft-expansion step queries only the newest nodes; the keys are
            the whole prefix and tree either way.

    Returns ``[n_tree - q_first, n_q_heads, head_dim]`` float64. For node ``i`` and head
    ``h`` with KV head ``g``: scores ``s_t = <q[i,h], K[g,t]> / sqrt(head_dim)``
    over the key set ``{0..prefix_len-1} U {prefix_len + j : j in anc*(i)}``,
    weights ``exp(s - max s)``, output the weighted mean of ``V[g, t]``.
    """
    par = check_parent(parent)
    q = _as_f64(q)
    _check_shapes(q, k_layer, v_layer, prefix_len, len(par), n_kv_heads, q_first)
    n, hq, d = q.shape
    group = hq // n_kv_heads
    scale = 1.0 / math.sqrt(d)
    out = np.empty((n, hq, d), dtype=np.float64)
    for r in range(n):
        i = q_first + r
        keys = list(range(prefix_len)) + [prefix_len + j for j in ancestors_inclusive(par, i)]
        for h in range(hq):
            g = h // group
            kk = _as_f64(k_layer[g, keys])
            vv = _as_f64(v_layer[g, keys])
            s = (kk @ q[r, h]) * scale
            w = np.exp(s - s.max())
            out[r, h] = (w @ vv) / w.sum()
    return out


def tree_attn_dense_ref(q, k_layer, v_layer, prefix_len, parent, n_kv_heads, q_first=0):
    """Same result as ``tree_attn_ref``, computed as dense masked softmax.

    The mask over the ``prefix_len + n_tree`` visible slots is all-True on the
    prefix and ``visibility_matrix(parent)`` on the tree block (its rows from
    ``q_first`` on). Masked scores are set to ``-inf`` before the softmax, so
    their weights are exactly 0.
    """
    par = check_parent(parent)
    q = _as_f64(q)
    _check_shapes(q, k_layer, v_layer, prefix_len, len(par), n_kv_heads, q_first)
    n, hq, d = q.shape
    group = hq // n_kv_heads
    total = prefix_len + len(par)
    mask = np.ones((n, total), dtype=bool)
    mask[:, prefix_len:] = visibility_matrix(par)[q_first:]
    out = np.empty((n, hq, d), dtype=np.float64)
    for g in range(n_kv_heads):
        kk = _as_f64(k_layer[g, :total])
        vv = _as_f64(v_layer[g, :total])
        qg = q[:, g * group:(g + 1) * group, :]                  # [n, G, d]
        s = np.matmul(qg, kk.T) / math.sqrt(d)                   # [n, G, total]
        s = np.where(mask[:, None, :], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        w = np.exp(s)
        w = w / w.sum(axis=-1, keepdims=True)
        out[:, g * group:(g + 1) * group, :] = np.matmul(w, vv)
    return out
