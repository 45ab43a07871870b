"""Greedy verification of a draft tree: which drafted tokens the target accepts.

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
may import this module.

Source: SwiftSpec (arXiv 2506.11309), Pith review page. "What carries the
argument" and the referee report's summary describe the loop this step sits
in: the target model checks the whole draft tree at once, the verified tokens
join the prefix and the draft tree is re-rooted at the last verified token.
Tree verification itself follows SpecInfer (the tree-based verification paper
in the page's reference list): every tree node is scored by the target in one
pass, so the target's next-token distribution is known at the virtual root
and at every node.

The pages do not state the acceptance rule. Taken here (greedy decoding,
temperature 0):

* the target's choice at a position is the arg-max of its logits there, the
  lowest token id among equal maxima (the values compared exactly as stored;
  -0.0 and +0.0 are equal);
* node ``i`` matches when its drafted token equals the target's choice at its
  parent (at the virtual root, logits row 0, when ``parent[i] == -1``);
* a node is accepted when it and every ancestor match; the accepted path is
  the root path of the deepest accepted node (the lowest index among equally
  deep ones), so ``m`` is its depth, or 0 when no first-level node matches;
* the bonus token is the target's choice at the last accepted node (at the
  virtual root when ``m == 0``): the token the target emits after the
  accepted ones.

Logits rows: row 0 is the virtual root (the last verified token), row
``1 + i`` is tree node ``i``.
"""

import numpy as np

from .tree_attn_ref import ancestors_inclusive, check_parent


def row_argmax(logits):
    """Per-row arg-max over exact values, lowest index on ties.

    ``logits`` [rows, vocab] of any real dtype; the upcast to float64 is exact
    for bf16 and fp32, so the comparison is the one the stored values give.
    ``numpy.argmax`` returns the first of equal maxima, and compares -0.0 and
    +0.0 as equal.
    """
    x = np.asarray(logits, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] < 1:
        raise ValueError("logits must be [rows, vocab] with vocab >= 1")
    return np.argmax(x, axis=1).astype(np.int64)


def tree_verify_ref(logits, tokens, parent):
    """Accepted path, bonus token and per-row target choices of one tree.

    ``logits`` [n + 1, vocab]; ``tokens`` [n] drafted token ids; ``parent``
    as for ``tree_attn_ref``. Returns ``(path, bonus, choice)``: ``path`` the
    accepted nodes root to leaf (a list, possibly empty), ``bonus`` an int,
    ``choice`` the per-row arg-max [n + 1].
    """
    par = check_parent(parent)
    n = len(par)
    x = np.asarray(logits)
    if x.ndim != 2 or x.shape[0] != n + 1:
        raise ValueError("logits must have n_tree + 1 rows")
    tok = [int(t) for t in tokens]
    if len(tok) != n:
        raise ValueError("one drafted token per tree node")
    choice = row_argmax(x)

    def target_choice_before(i):
        return int(choice[0 if par[i] < 0 else 1 + par[i]])

    matches = [tok[i] == target_choice_before(i) for i in range(n)]
    best, best_depth = -1, 0
    for i in range(n):
        chain = ancestors_inclusive(par, i)
        if all(matches[a] for a in chain) and len(chain) > best_depth:
            best, best_depth = i, len(chain)  # strict '>' keeps the lowest index
    path = sorted(ancestors_inclusive(par, best)) if best >= 0 else []
    bonus = int(choice[0 if best < 0 else 1 + best])
    return path, bonus, choice
