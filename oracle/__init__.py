"""CPU fp64 oracle for tree-masked attention and KV-cache re-rooting.

This package is TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``tree_masked_attention_attn_amd``) never imports, calls or links anything here,
and nothing here imports the product path: the two share no code.

What the oracle computes follows the SwiftSpec pages (arXiv 2506.11309, the
Pith review page), sections "What carries the argument" and "Core claim":

* the draft KV cache holds the verified tokens as a contiguous prefix with the
  draft-tree tokens right after it, and attention over the tree is masked so
  that each tree token sees the prefix plus its own root path
  (``tree_attn_ref`` / ``tree_attn_dense_ref``);
* after verification the tree is re-rooted at the last verified token: the
  accepted tokens join the prefix and the surviving subtree is laid out
  contiguously after it (``kv_reroot_ref``).

Every function is a plain definition in float64 (attention) or a byte-exact
gather (re-root). Points the pages leave open are taken as follows:

* a node attends to itself and to all of its ancestors;
* ``parent[i] == -1`` means the node hangs off the last prefix token, so a
  forest of first-level nodes is allowed;
* the softmax scale is ``1/sqrt(head_dim)``;
* query head ``h`` reads KV head ``h // (n_q_heads // n_kv_heads)``;
* the whole accepted path moves into the prefix; survivors keep ascending
  original order.

Maximum-likelihood expansion (``tree_expand_ref``): the k best (leaf, token)
candidates by path score plus log-softmax become the new nodes.

Tree verification (``tree_verify_ref``) reads the acceptance rule as greedy:
a drafted token is accepted when it equals the target's arg-max at its parent
and every ancestor was accepted; the deepest such node ends the accepted path.

Parity pinning: every function here is pinned by ``-m "not gpu"`` tests
against torch's CPU ``scaled_dot_product_attention`` (causal and decode special
cases), hand-derived golden fixtures, closed forms and brute force over all
trees of up to six nodes; verification against a top-down walk of the tree
that consumes the target's tokens one at a time. No function is "parity unpinned".
"""

from .tree_attn_ref import (  # noqa: F401
    ancestors_inclusive,
    check_parent,
    tree_attn_ref,
    tree_attn_dense_ref,
    visibility_matrix,
)
from .kv_reroot_ref import check_reroot_args, kv_reroot_ref, reroot_plan_ref  # noqa: F401
from .tree_verify_ref import row_argmax, tree_verify_ref  # noqa: F401
from .tree_expand_ref import log_softmax_rows, token_ranking, tree_expand_ref  # noqa: F401
