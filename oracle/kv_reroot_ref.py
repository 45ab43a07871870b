"""KV-cache re-root and compaction, written out as a byte-exact gather.

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
may import this module.

Source: SwiftSpec (arXiv 2506.11309), Pith review page. "What carries the
argument" says the draft tree is re-rooted at the last verified token after each
verification and the cache is reorganised to keep only the subtree that is
still useful. "Core claim" says verified tokens are moved into the prefix cache
and the surviving tree states are laid out contiguously after it. The referee
summary adds that partially rejected branches are reused.

Readings taken where the pages are silent:

* the whole accepted path ``a_0 .. a_{m-1}`` (root to leaf order) joins the
  prefix, so the new prefix length is ``prefix_len + m``;
* the survivors are the caller's choice: any set of strict descendants of
  ``a_{m-1}`` closed under ``parent`` (with ``m == 0`` their tops hang off the
  virtual root); they are kept in ascending original index, which keeps
  ``parent[i] < i`` and makes the result unique;
* cache slots at or beyond ``prefix_len + m + len(survivors)`` are left as they
  were (nothing is cleared).
"""

import numpy as np

from .tree_attn_ref import check_parent


def check_reroot_args(prefix_len, parent, path, survivors, capacity):
    """Validate a re-root request; raise ``ValueError`` on anything malformed.

    * ``path`` is a chain from a first-level node downward:
      ``parent[a_0] == -1`` and ``parent[a_k] == a_{k-1}``;
    * ``survivors`` is strictly ascending, disjoint from ``path``, and closed
      under ``parent`` with tops attached to ``a_{m-1}`` (or to -1 when the path
      is empty);
    * ``prefix_len + n_tree <= capacity``.
    """
    par = check_parent(parent)
    n = len(par)
    path = [int(a) for a in path]
    surv = [int(s) for s in survivors]
    if prefix_len < 0 or prefix_len + n > capacity:
        raise ValueError("prefix_len + n_tree exceeds capacity")
    for a in path + surv:
        if not 0 <= a < n:
            raise ValueError(f"node {a} out of range")
    for k, a in enumerate(path):
        want = -1 if k == 0 else path[k - 1]
        if par[a] != want:
            raise ValueError(f"accepted path breaks at position {k}")
    for k in range(1, len(surv)):
        if surv[k] <= surv[k - 1]:
            raise ValueError("survivors must be strictly ascending")
    if set(surv) & set(path):
        raise ValueError("a survivor is on the accepted path")
    last = path[-1] if path else -1
    allowed = set(surv) | {last}
    for s in surv:
        if par[s] not in allowed:
            raise ValueError(f"survivor {s} is not below the last accepted node")
    return par, path, surv


def reroot_plan_ref(prefix_len, parent, path, survivors, capacity):
    """Return ``(order, new_prefix_len, new_parent)`` for a re-root request.

    ``order`` lists the old tree indices in their new slot order: the accepted
    path first (it becomes prefix slots ``prefix_len .. prefix_len+m-1``), then
    the survivors (new tree nodes ``0 .. len(survivors)-1``). ``new_parent[k]``
    is -1 when survivor ``k`` hung directly off the last accepted node,
    otherwise the new index of its parent among the survivors.
    """
    par, path, surv = check_reroot_args(prefix_len, parent, path, survivors, capacity)
    last = path[-1] if path else -1
    new_index = {s: k for k, s in enumerate(surv)}
    new_parent = [-1 if par[s] == last else new_index[par[s]] for s in surv]
    return path + surv, prefix_len + len(path), new_parent


def kv_reroot_ref(k_cache, v_cache, prefix_len, parent, path, survivors):
    """Re-root every layer and KV head of a cache; returns new arrays.

    ``k_cache`` and ``v_cache`` are ``[n_layers, n_kv_heads, capacity, head_dim]``
    arrays of any dtype (bf16 caches are passed as their raw 16-bit words), so
    the result is byte-exact by construction: slot ``prefix_len + k`` of the
    result receives the old slot ``prefix_len + order[k]``; every other slot
    keeps its old bytes.

    Returns ``(k_new, v_new, new_prefix_len, new_parent)``.
    """
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    if k_cache.ndim != 4 or k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k and v caches must be [n_layers, n_kv_heads, capacity, head_dim] alike")
    order, new_prefix, new_parent = reroot_plan_ref(
        prefix_len, parent, path, survivors, k_cache.shape[2])
    k_new = k_cache.copy()
    v_new = v_cache.copy()
    src = [prefix_len + o for o in order]
    dst = slice(prefix_len, prefix_len + len(order))
    k_new[:, :, dst] = k_cache[:, :, src]
    v_new[:, :, dst] = v_cache[:, :, src]
    return k_new, v_new, new_prefix, new_parent
