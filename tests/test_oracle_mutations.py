"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

A pin that cannot tell a correct oracle from a broken one pins nothing. Each
mutant below is the oracle with one realistic slip; the test asserts that at
least one pin reports an error far above its tolerance.
"""

import importlib
import itertools
import os
import math

import numpy as np
import pytest

import oracle
from tests import pins

attn_mod = importlib.import_module("oracle.tree_attn_ref")
reroot_mod = importlib.import_module("oracle.kv_reroot_ref")


def attention_pins(attn):
    rng = np.random.default_rng(5)
    errs = [
        pins.pin_chain_causal(attn, rng),
        pins.pin_root_only_decode(attn, rng),
        pins.pin_golden_uniform(attn, rng),
    ]
    for parent in ([-1, 0, 0, 1, -1, 4, 3], [-1, -1, 1, 2]):
        for x in range(len(parent)):
            errs.append(pins.pin_path_reroot_causal(attn, oracle.kv_reroot_ref, parent, x, rng))
    return max(errs)


def test_unmutated_oracle_passes_every_pin():
    assert attention_pins(oracle.tree_attn_ref) < 1e-12
    assert attention_pins(oracle.tree_attn_dense_ref) < 1e-12


def _no_self(parent, i):
    return [a for a in _orig_anc(parent, i) if a != i]


def _stop_below_root(parent, i):
    chain = _orig_anc(parent, i)
    return chain[1:] if len(chain) > 1 else chain


def _with_parent_of_parent_only(parent, i):
    # skips every other ancestor
    return [a for k, a in enumerate(reversed(_orig_anc(parent, i))) if k % 2 == 0]


_orig_anc = attn_mod.ancestors_inclusive


@pytest.mark.parametrize("bad", [_no_self, _stop_below_root, _with_parent_of_parent_only])
def test_wrong_ancestor_walk_is_caught(monkeypatch, bad):
    monkeypatch.setattr(attn_mod, "ancestors_inclusive", bad)
    assert attention_pins(oracle.tree_attn_ref) > 1e-3


def test_visibility_without_diagonal_is_caught(monkeypatch):
    orig = attn_mod.visibility_matrix

    def bad(parent):
        m = orig(parent).copy()
        np.fill_diagonal(m, False)
        return m
    monkeypatch.setattr(attn_mod, "visibility_matrix", bad)
    with np.errstate(invalid="ignore"):
        err = attention_pins(oracle.tree_attn_dense_ref)
    assert not err < 1e-3


def test_visibility_one_step_only_is_caught(monkeypatch):
    """Forgetting the transitive closure leaves only parent and self visible."""
    def bad(parent):
        n = len(parent)
        m = np.eye(n, dtype=bool)
        for i, p in enumerate(parent):
            if p >= 0:
                m[i, p] = True
        return m
    monkeypatch.setattr(attn_mod, "visibility_matrix", bad)
    assert attention_pins(oracle.tree_attn_dense_ref) > 1e-3


def test_missing_score_scale_is_caught():
    def bad(q, k, v, P, parent, hkv):
        return oracle.tree_attn_ref(np.asarray(q) * math.sqrt(np.shape(q)[-1]), k, v, P, parent, hkv)
    assert attention_pins(bad) > 1e-3


def test_wrong_gqa_head_mapping_is_caught():
    def bad(q, k, v, P, parent, hkv):
        hq = np.shape(q)[1]
        idx = [h % hkv for h in range(hq)]
        return oracle.tree_attn_ref(q, np.asarray(k)[idx], np.asarray(v)[idx], P, parent, hq)
    assert attention_pins(bad) > 1e-3


def test_swapped_key_and_value_is_caught():
    def bad(q, k, v, P, parent, hkv):
        return oracle.tree_attn_ref(q, v, k, P, parent, hkv)
    assert attention_pins(bad) > 1e-3


def test_prefix_off_by_one_is_caught():
    """Dropping the last prefix key (a range bound slip)."""
    def bad(q, k, v, P, parent, hkv):
        q = np.asarray(q, dtype=np.float64)
        n, hq, d = q.shape
        out = np.empty_like(q)
        for i in range(n):
            keys = list(range(max(P - 1, 0))) + [P + j for j in oracle.ancestors_inclusive(parent, i)]
            for h in range(hq):
                g = h // (hq // hkv)
                s = np.asarray(k)[g, keys] @ q[i, h] / math.sqrt(d)
                w = np.exp(s - s.max())
                out[i, h] = w @ np.asarray(v)[g, keys] / w.sum()
        return out
    assert attention_pins(bad) > 1e-3


def test_frontier_rows_taken_from_the_wrong_nodes_are_caught():
    """Frontier queries placed on the first tree nodes, or one node early."""
    assert pins.pin_chain_frontier_causal(oracle.tree_attn_ref, np.random.default_rng(6)) < 1e-12

    def first_nodes(q, k, v, P, parent, hkv, q_first=0):
        n, w = len(parent), len(parent) - q_first
        qq = np.zeros((n,) + np.shape(q)[1:])
        qq[:w] = q
        return oracle.tree_attn_dense_ref(qq, k, v, P, parent, hkv)[:w]

    def one_early(q, k, v, P, parent, hkv, q_first=0):
        n, w = len(parent), len(parent) - q_first
        qq = np.zeros((n,) + np.shape(q)[1:])
        qq[q_first - 1:n - 1] = q
        return oracle.tree_attn_dense_ref(qq, k, v, P, parent, hkv)[q_first - 1:n - 1]

    for bad in (first_nodes, one_early):
        assert pins.pin_chain_frontier_causal(bad, np.random.default_rng(6)) > 1e-3


def test_reroot_plan_slips_are_caught(monkeypatch):
    assert pins.pin_reroot_golden(oracle.reroot_plan_ref) == 0
    orig = reroot_mod.reroot_plan_ref

    def parent_off_by_one(*a):
        order, p, par = orig(*a)
        return order, p, [x + 1 if x >= 0 else x for x in par]

    def survivors_reversed(*a):
        order, p, par = orig(*a)
        m = p - a[0]
        return order[:m] + order[m:][::-1], p, par

    def path_not_in_prefix(*a):
        order, p, par = orig(*a)
        return order, a[0], par

    for bad in (parent_off_by_one, survivors_reversed, path_not_in_prefix):
        assert pins.pin_reroot_golden(bad) > 0


def test_reroot_gather_slip_is_caught(monkeypatch):
    """A gather that leaves the accepted path where it was breaks the causal pin."""
    def bad_reroot(k, v, P, parent, path, surv):
        k2, v2, new_p, new_par = oracle.kv_reroot_ref(k, v, P, parent, path, surv)
        k2[:, :, P] = k[:, :, P]
        v2[:, :, P] = v[:, :, P]
        return k2, v2, new_p, new_par
    rng = np.random.default_rng(9)
    parent = [-1, -1, 1, 2]
    errs = [pins.pin_path_reroot_causal(oracle.tree_attn_ref, bad_reroot, parent, x, rng) for x in range(4)]
    assert max(errs) > 1e-3


# ---------------------------------------------------------------------------
# Tree verification: each mutant is the oracle's source with one slip.

_VERIFY_SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                "oracle", "tree_verify_ref.py")).read()


def _verify_mutant(old, new):
    assert _VERIFY_SRC.count(old) == 1, old
    ns = {"__name__": "oracle.tree_verify_mutant", "__package__": "oracle"}
    exec(compile(_VERIFY_SRC.replace(old, new), "tree_verify_mutant", "exec"), ns)
    return ns["tree_verify_ref"]


def verify_pins(verify):
    rng = np.random.default_rng(9)
    parents = [list(p) for n in (3, 4) for p in itertools.product(*[range(-1, i) for i in range(n)])]
    return (pins.pin_verify_golden(verify) + pins.pin_verify_walk(verify, parents, rng)
            + pins.pin_verify_chain(verify, rng))


def test_unmutated_verify_passes_every_pin():
    assert verify_pins(oracle.tree_verify_ref) == 0


VERIFY_SLIPS = {
    "own_row_instead_of_parent_row": ("0 if par[i] < 0 else 1 + par[i]", "1 + i"),
    "matches_without_ancestors": ("all(matches[a] for a in chain)", "matches[i]"),
    "ties_to_highest_index": ("len(chain) > best_depth", "len(chain) >= best_depth"),
    "bonus_from_parent_row": ("bonus = int(choice[0 if best < 0 else 1 + best])",
                              "bonus = int(choice[0 if best < 0 else 1 + par[best]])"),
    "argmax_last_of_equal_maxima": ("return np.argmax(x, axis=1).astype(np.int64)",
                                    "return (x.shape[1] - 1 - np.argmax(x[:, ::-1], axis=1)).astype(np.int64)"),
    "path_leaf_to_root": ("path = sorted(ancestors_inclusive(par, best))",
                          "path = sorted(ancestors_inclusive(par, best), reverse=True)"),
    "argmax_on_bit_patterns": ("x = np.asarray(logits, dtype=np.float64)",
                               "x = np.asarray(logits, dtype=np.float32).view(np.int32).astype(np.float64)"),
}


@pytest.mark.parametrize("slip", list(VERIFY_SLIPS))
def test_verify_slip_is_caught(slip):
    assert verify_pins(_verify_mutant(*VERIFY_SLIPS[slip])) > 0


# ---------------------------------------------------------------------------
# Maximum-likelihood expansion: each mutant is the oracle's source with one slip.

_EXPAND_SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                "oracle", "tree_expand_ref.py")).read()


def _expand_mutant(old, new):
    assert _EXPAND_SRC.count(old) == 1, old
    ns = {"__name__": "oracle.tree_expand_mutant", "__package__": "oracle"}
    exec(compile(_EXPAND_SRC.replace(old, new), "tree_expand_mutant", "exec"), ns)
    return ns["tree_expand_ref"]


def expand_pins(expand):
    rng = np.random.default_rng(41)
    return max(pins.pin_expand_golden(expand), pins.pin_expand_bruteforce(expand, rng, trials=30),
               pins.pin_expand_uniform(expand, rng))


def test_unmutated_expand_passes_every_pin():
    assert expand_pins(oracle.tree_expand_ref) < 1e-12


EXPAND_SLIPS = {
    "no_path_score": ("cands.append((float(s[i] + logp[i, t])", "cands.append((float(logp[i, t])"),
    "probability_not_log": ("cands.append((float(s[i] + logp[i, t])", "cands.append((float(s[i] + np.exp(logp[i, t]))"),
    "raw_logits": ("logp = log_softmax_rows(x)", "logp = x"),
    "max_not_taken_out": ("return x - (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))",
                          "return x - np.log(np.exp(x).sum(axis=1, keepdims=True))"),
    "rank_ties_to_higher_id": ("return np.lexsort((np.arange(row.size), -row))",
                               "return np.lexsort((-np.arange(row.size), -row))"),
    "score_ties_to_higher_leaf": ("cands.sort(key=lambda c: (-c[0], c[1], c[2]))",
                                  "cands.sort(key=lambda c: (-c[0], -c[1], c[2]))"),
    "listed_by_score": ("chosen = sorted(cands[:k], key=lambda c: (c[1], c[2]))", "chosen = cands[:k]"),
    "one_candidate_per_leaf": ("enumerate(token_ranking(x[i])[:k])", "enumerate(token_ranking(x[i])[:1])"),
}


@pytest.mark.parametrize("slip", list(EXPAND_SLIPS))
def test_expand_slip_is_caught(slip):
    assert expand_pins(_expand_mutant(*EXPAND_SLIPS[slip])) > 1e-6
