"""Checks that tie the oracle to facts outside itself.

Each ``pin_*`` takes the attention (or re-root) function under test and returns
the worst deviation from something the oracle did not compute: torch's CPU
``scaled_dot_product_attention`` in the causal and decode special cases,
hand-derived golden sets, closed forms. ``test_oracle_pins.py`` runs them on the
oracle; ``test_oracle_mutations.py`` runs them on oracles with a planted
mistake and expects them to fail.
"""

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand(rng, *shape):
    return rng.standard_normal(shape)


def sdpa_causal(q_seq, k_seq, v_seq):
    """Causal self-attention over a whole sequence, by torch (fp64, CPU).

    q_seq: [L, Hq, d]; k_seq, v_seq: [L, Hkv, d]. Returns [L, Hq, d].
    """
    q = torch.from_numpy(q_seq).permute(1, 0, 2)[None]
    k = torch.from_numpy(k_seq).permute(1, 0, 2)[None]
    v = torch.from_numpy(v_seq).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def sdpa_full(q_rows, k_seq, v_seq):
    """Unmasked attention of a few query rows over a key sequence, by torch.

    q_rows: [n, Hq, d]; k_seq, v_seq: [L, Hkv, d].
    """
    q = torch.from_numpy(q_rows).permute(1, 0, 2)[None]
    k = torch.from_numpy(k_seq).permute(1, 0, 2)[None]
    v = torch.from_numpy(v_seq).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(q, k, v, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def chain_parent(n):
    return [-1] + list(range(n - 1))


def pin_chain_causal(attn, rng, prefix_len=37, n=9, hq=8, hkv=2, d=16):
    """A chain tree is the tail of an ordinary causal sequence.

    The tree tokens are the last ``n`` tokens of a sequence of length
    ``prefix_len + n``; their outputs must equal torch's causal attention there.
    """
    L = prefix_len + n
    q_seq = rand(rng, L, hq, d)
    k_seq = rand(rng, L, hkv, d)
    v_seq = rand(rng, L, hkv, d)
    want = sdpa_causal(q_seq, k_seq, v_seq)[prefix_len:]
    cap = L + 5
    k = np.full((hkv, cap, d), np.nan)
    v = np.full((hkv, cap, d), np.nan)
    k[:, :L] = k_seq.transpose(1, 0, 2)
    v[:, :L] = v_seq.transpose(1, 0, 2)
    got = attn(q_seq[prefix_len:], k, v, prefix_len, chain_parent(n), hkv)
    return float(np.abs(got - want).max())


def pin_chain_frontier_causal(attn, rng, prefix_len=29, n=12, w=4, hq=4, hkv=2, d=8):
    """Frontier-only queries on a chain tree are the last rows of causal attention.

    Only the newest ``w`` nodes of the chain have queries (``q_first = n - w``);
    the keys are the whole prefix and chain, so those rows must equal torch's
    causal attention over the sequence of length ``prefix_len + n`` at its
    last ``w`` positions.
    """
    L = prefix_len + n
    q_seq = rand(rng, L, hq, d)
    k_seq = rand(rng, L, hkv, d)
    v_seq = rand(rng, L, hkv, d)
    want = sdpa_causal(q_seq, k_seq, v_seq)[L - w:]
    cap = L + 3
    k = np.full((hkv, cap, d), np.nan)
    v = np.full((hkv, cap, d), np.nan)
    k[:, :L] = k_seq.transpose(1, 0, 2)
    v[:, :L] = v_seq.transpose(1, 0, 2)
    got = attn(q_seq[L - w:], k, v, prefix_len, chain_parent(n), hkv, q_first=n - w)
    return float(np.abs(got - want).max())


def pin_root_only_decode(attn, rng, prefix_len=50, hq=4, hkv=4, d=32):
    """A single node under the virtual root is plain one-token decode attention."""
    L = prefix_len + 1
    q = rand(rng, 1, hq, d)
    k_seq = rand(rng, L, hkv, d)
    v_seq = rand(rng, L, hkv, d)
    want = sdpa_full(q, k_seq, v_seq)
    got = attn(q, k_seq.transpose(1, 0, 2).copy(), v_seq.transpose(1, 0, 2).copy(),
               prefix_len, [-1], hkv)
    return float(np.abs(got - want).max())


def pin_golden_uniform(attn, rng, prefix_len=6, hq=2, hkv=1, d=8):
    """With zero queries every visible key weighs the same, so each output is the
    plain mean of the visible value rows; the visible sets come from the
    hand-derived golden file."""
    worst = 0.0
    for case in load_golden("mask_visible_sets.json")["cases"]:
        parent = case["parent"]
        n = len(parent)
        cap = prefix_len + n + 3
        k = rand(rng, hkv, cap, d)
        v = rand(rng, hkv, cap, d)
        k[:, prefix_len + n:] = np.nan
        v[:, prefix_len + n:] = np.nan
        q = np.zeros((n, hq, d))
        got = attn(q, k, v, prefix_len, parent, hkv)
        for i, vis in enumerate(case["visible"]):
            rows = list(range(prefix_len)) + [prefix_len + j for j in vis]
            for h in range(hq):
                want = v[h // (hq // hkv), rows].mean(axis=0)
                worst = max(worst, float(np.abs(got[i, h] - want).max()))
    return worst


def pin_path_reroot_causal(attn, reroot, parent, x, rng, prefix_len=5, hq=4, hkv=2, d=8):
    """Node ``x`` of any tree sees exactly what the last token of a causal
    sequence sees once its root path has been moved into the prefix.

    The root path of ``x`` is found here by its own walk; the re-root (a pure
    gather) lays the path out as prefix rows; torch's causal attention over that
    new prefix then gives ``x``'s output at the last position.
    """
    n = len(parent)
    path = [x]
    while parent[path[-1]] != -1:
        path.append(parent[path[-1]])
    path.reverse()
    cap = prefix_len + n + 2
    k = rand(rng, 1, hkv, cap, d)
    v = rand(rng, 1, hkv, cap, d)
    q = rand(rng, n, hq, d)
    got = attn(q, k[0], v[0], prefix_len, parent, hkv)[x]
    k2, v2, new_p, _ = reroot(k, v, prefix_len, parent, path, [])
    L = new_p
    q_seq = np.zeros((L, hq, d))
    q_seq[-1] = q[x]
    want = sdpa_causal(q_seq, k2[0, :, :L].transpose(1, 0, 2).copy(),
                       v2[0, :, :L].transpose(1, 0, 2).copy())[-1]
    return float(np.abs(got - want).max())


def pin_reroot_golden(plan):
    """Hand-worked re-root cases: returns the number of mismatching cases.

    ``plan(prefix_len, parent, path, survivors, capacity)`` returns
    ``(order, new_prefix_len, new_parent)``.
    """
    bad = 0
    for case in load_golden("reroot_cases.json")["cases"]:
        cap = case["prefix_len"] + len(case["parent"])
        order, new_p, new_par = plan(case["prefix_len"], case["parent"], case["path"],
                                     case["survivors"], cap)
        src = [case["prefix_len"] + o for o in order]
        dst = [case["prefix_len"] + k for k in range(len(order))]
        if (list(order) != case["order"] or src != case["src_slots"] or dst != case["dst_slots"]
                or new_p != case["new_prefix_len"] or list(new_par) != case["new_parent"]):
            bad += 1
    return bad


def scale_of(d):
    return 1.0 / math.sqrt(d)


# ---------------------------------------------------------------------------
# Tree verification (greedy acceptance). The pins below compute the target's
# choices with a plain loop and find the accepted path by walking DOWN from
# the virtual root along matching children, the way speculative decoding
# consumes the target's tokens one at a time; the oracle instead checks every
# node's root path bottom-up.


def loop_argmax(row):
    """First index of the maximum, by a plain scan (-0.0 == +0.0 as floats)."""
    best = 0
    for j in range(1, len(row)):
        if float(row[j]) > float(row[best]):
            best = j
    return best


def walk_accepted(choice, tokens, parent):
    """Deepest node reachable from the virtual root through matching children.

    Explores every matching child (siblings may share a token), so the result
    is the deepest such node, the lowest index among equally deep ones.
    """
    n = len(parent)
    children = {-1: []}
    for i in range(n):
        children.setdefault(i, [])
        children[int(parent[i])].append(i)
    best = (0, 0, [])  # (depth, -index, path)
    stack = [(-1, [])]
    while stack:
        node, path = stack.pop()
        want = choice[0 if node < 0 else 1 + node]
        for c in children[node]:
            if int(tokens[c]) == want:
                p = path + [c]
                if (len(p), -c) > best[:2]:
                    best = (len(p), -c, p)
                stack.append((c, p))
    path = best[2]
    bonus = choice[0 if not path else 1 + path[-1]]
    return path, bonus


def golden_verify_cases():
    cases = load_golden("verify_cases.json")["cases"]
    for c in cases:
        c = dict(c)
        c["logits"] = np.array([[float(v) for v in row] for row in c["logits"]], dtype=np.float32)
        yield c


def pin_verify_golden(verify):
    """Number of hand-worked cases whose path, bonus or choices differ."""
    bad = 0
    for c in golden_verify_cases():
        path, bonus, choice = verify(c["logits"], c["tokens"], c["parent"])
        bad += (list(path) != c["path"]) or (int(bonus) != c["bonus"]) or (list(map(int, choice)) != c["choice"])
    return bad


def pin_verify_walk(verify, parents, rng, vocab=3, draws=3):
    """Mismatches against the top-down walk over the given trees.

    Logits are small integers (many equal maxima) and tokens come from a tiny
    vocabulary (siblings often share one), so ties decide many cases.
    """
    bad = 0
    for parent in parents:
        n = len(parent)
        for _ in range(draws):
            logits = rng.integers(-2, 3, size=(n + 1, vocab)).astype(np.float32)
            choice = [loop_argmax(r) for r in logits]
            # bias tokens toward the target's choice so paths get long
            tokens = [choice[0 if parent[i] < 0 else 1 + parent[i]] if rng.random() < 0.7
                      else int(rng.integers(0, vocab)) for i in range(n)]
            want_path, want_bonus = walk_accepted(choice, tokens, parent)
            path, bonus, got_choice = verify(logits, tokens, parent)
            bad += (list(path) != want_path) or (int(bonus) != want_bonus) or (list(map(int, got_choice)) != choice)
    return bad


def pin_verify_chain(verify, rng, n=12, vocab=50):
    """Chain tree whose drafted tokens agree with the target for exactly k
    steps: the accepted length is k and the bonus is the target's choice at
    node k - 1 (a planted unique maximum per row)."""
    bad = 0
    parent = chain_parent(n)
    for k in range(n + 1):
        planted = rng.integers(0, vocab, size=n + 1)
        logits = rng.standard_normal((n + 1, vocab)).astype(np.float32)
        logits[np.arange(n + 1), planted] = 10.0
        tokens = [int(planted[i]) for i in range(n)]  # node i follows row i
        if k < n:
            tokens[k] = int((planted[k] + 1) % vocab)
        path, bonus, _ = verify(logits, tokens, parent)
        bad += (list(path) != list(range(k))) or (int(bonus) != int(planted[k]))
    return bad


# ---------------------------------------------------------------------------
# Maximum-likelihood expansion. The pins use scipy's log_softmax (a library
# routine) and rank EVERY candidate of every leaf in one global sort; the
# oracle keeps only each leaf's k best tokens before merging.


def golden_expand_cases():
    for c in load_golden("expand_cases.json")["cases"]:
        c = dict(c)
        with np.errstate(divide="ignore"):
            x = np.log(np.array(c["weights"], dtype=np.float64))
            c["path_scores"] = np.log(np.array(c["path_prob"], dtype=np.float64))
        if "offsets" in c:
            x = x + np.array(c["offsets"])[:, None]
        c["logits"] = x
        yield c


def pin_expand_golden(expand):
    """Worst deviation over the hand-worked cases: inf on a wrong node list,
    else the largest score error."""
    worst = 0.0
    for c in golden_expand_cases():
        got = expand(c["logits"], c["path_scores"], c["k"])
        if [(int(i), int(t)) for i, t, _ in got] != [(i, t) for i, t, _ in c["nodes"]]:
            return math.inf
        for (_, _, s), (_, _, p) in zip(got, c["nodes"]):
            want = math.log(p) if p > 0 else -math.inf
            err = 0.0 if s == want else abs(s - want)
            worst = max(worst, err)
    return worst


def expand_bruteforce(logits, path_scores, k):
    """Every (leaf, token) of every leaf, scored with scipy's log_softmax and
    ranked in one sort."""
    from scipy.special import log_softmax
    x = np.asarray(logits, dtype=np.float64)
    logp = log_softmax(x, axis=1)
    w, vocab = x.shape
    every = []
    for i in range(w):
        by_logit = sorted(range(vocab), key=lambda t: (-x[i, t], t))
        for slot, t in enumerate(by_logit):
            every.append((path_scores[i] + logp[i, t], i, slot, t))
    every.sort(key=lambda c: (-c[0], c[1], c[2]))
    return [(i, t, s) for s, i, slot, t in sorted(every[:k], key=lambda c: (c[1], c[2]))]


def pin_expand_bruteforce(expand, rng, trials=60):
    """Worst deviation from the global brute force on small random frontiers
    (integer logits, so equal logits and equal scores are common)."""
    worst = 0.0
    for _ in range(trials):
        w, vocab = int(rng.integers(1, 7)), int(rng.integers(1, 41))
        k = int(rng.integers(1, min(w * vocab, 20) + 1))
        if rng.random() < 0.5:
            x = rng.integers(-3, 4, size=(w, vocab)).astype(np.float64)
            s = rng.integers(-2, 1, size=w).astype(np.float64)
        else:
            x = rng.standard_normal((w, vocab)) * 3
            s = -rng.random(w) * 4
        got = expand(x, s, k)
        want = expand_bruteforce(x, s, k)
        if [(int(i), int(t)) for i, t, _ in got] != [(i, t) for i, t, _ in want]:
            return math.inf
        worst = max(worst, max(abs(a[2] - b[2]) for a, b in zip(got, want)))
    return worst


def pin_expand_uniform(expand, rng):
    """Equal logits within each row: every token of leaf i scores
    s[i] - ln(vocab); leaves are taken by descending path score, tokens in
    id order."""
    worst = 0.0
    for w, vocab, k in ((3, 5, 7), (8, 16, 8), (1, 9, 9), (4, 2, 8)):
        s = -rng.permutation(w).astype(np.float64) * 0.75  # distinct
        x = np.repeat(rng.standard_normal((w, 1)), vocab, axis=1)
        want = []
        for i in np.argsort(-s):
            for t in range(vocab):
                if len(want) < k:
                    want.append((int(i), t, s[i] - math.log(vocab)))
        want.sort()
        got = expand(x, s, k)
        if [(int(i), int(t)) for i, t, _ in got] != [(i, t) for i, t, _ in want]:
            return math.inf
        worst = max(worst, max(abs(a[2] - b[2]) for a, b in zip(got, want)))
    return worst
