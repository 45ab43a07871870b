"""Maximum-likelihood expansion of a draft tree by k new nodes.

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
may import this module.

Source: SwiftSpec (arXiv 2506.11309), Pith review page, "Assumptions & free
parameters": the draft tree grows by maximum likelihood, a path's score being
the sum of the log-softmax probabilities of its tokens, with expansion width
w = 8; "What carries the argument": the draft model expands the tree while
the target verifies the previous one.

One expansion step, as read here (the pages give no listing of it):

* the frontier is ``w`` leaves; leaf ``i`` has path score ``s[i]`` and the
  draft model's logits ``x[i]`` over the vocabulary for the token after it;
* every (leaf, token) pair is a candidate child with score
  ``s[i] + log_softmax(x[i])[token]``;
* the ``k`` best candidates become new nodes. A leaf's own candidates are
  ranked by logit (the lower token id first among equal logits), and that
  rank is the child's slot; equal scores are broken by the lower leaf, then
  the lower slot;
* the new nodes are listed by (leaf, slot), the order the tree generator of
  the workloads also uses for the nodes of one round.

Returns ``[(leaf, token, score), ...]``.
"""

import numpy as np


def log_softmax_rows(x):
    """``x - logsumexp(x)`` per row in float64, with the row maximum taken out
    first so that large logits do not overflow. ``-inf`` entries are allowed
    (probability 0); a row needs at least one finite value."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=1, keepdims=True)
    if not np.isfinite(m).all():
        raise ValueError("every row needs a finite maximum")
    return x - (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))


def token_ranking(row):
    """Token ids of one row by descending logit, the lower id first on ties."""
    row = np.asarray(row, dtype=np.float64)
    return np.lexsort((np.arange(row.size), -row))


def tree_expand_ref(logits, path_scores, k):
    """The ``k`` new nodes of one maximum-likelihood expansion step.

    ``logits`` [w, vocab] (any real dtype; exact upcast), ``path_scores`` [w].
    A leaf can give at most ``k`` of the new nodes, so only each leaf's ``k``
    best tokens are candidates.
    """
    x = np.asarray(logits, dtype=np.float64)
    if x.ndim != 2 or x.shape[0] < 1 or x.shape[1] < 1:
        raise ValueError("logits must be [w, vocab] with w, vocab >= 1")
    s = np.asarray(path_scores, dtype=np.float64)
    w, vocab = x.shape
    if s.shape != (w,):
        raise ValueError("one path score per frontier leaf")
    if not 1 <= k <= w * vocab:
        raise ValueError("k must be in [1, w * vocab]")
    logp = log_softmax_rows(x)
    cands = []
    for i in range(w):
        for slot, t in enumerate(token_ranking(x[i])[:k]):
            cands.append((float(s[i] + logp[i, t]), i, slot, int(t)))
    cands.sort(key=lambda c: (-c[0], c[1], c[2]))
    chosen = sorted(cands[:k], key=lambda c: (c[1], c[2]))
    return [(i, t, score) for score, i, slot, t in chosen]
