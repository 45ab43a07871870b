"""Pins of the CPU oracle against facts it did not compute itself (CPU only)."""

import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests import pins

TIGHT = 1e-12


@pytest.mark.parametrize("attn", [oracle.tree_attn_ref, oracle.tree_attn_dense_ref])
@pytest.mark.parametrize("shape", [(37, 9, 8, 2, 16), (1, 1, 1, 1, 4), (64, 33, 4, 4, 8), (0, 5, 6, 3, 8)])
def test_chain_tree_is_causal_attention(attn, shape):
    P, n, hq, hkv, d = shape
    rng = np.random.default_rng(11)
    assert pins.pin_chain_causal(attn, rng, P, n, hq, hkv, d) < TIGHT


@pytest.mark.parametrize("attn", [oracle.tree_attn_ref, oracle.tree_attn_dense_ref])
@pytest.mark.parametrize("shape", [(50, 4, 4, 32), (1, 2, 1, 8), (0, 8, 2, 16)])
def test_root_only_tree_is_decode_attention(attn, shape):
    P, hq, hkv, d = shape
    rng = np.random.default_rng(12)
    assert pins.pin_root_only_decode(attn, rng, P, hq, hkv, d) < TIGHT


def test_visible_sets_match_hand_derived_golden():
    for case in pins.load_golden("mask_visible_sets.json")["cases"]:
        parent = case["parent"]
        vis = oracle.visibility_matrix(parent)
        for i, want in enumerate(case["visible"]):
            assert oracle.ancestors_inclusive(parent, i) == want
            assert sorted(np.nonzero(vis[i])[0].tolist()) == want


@pytest.mark.parametrize("attn", [oracle.tree_attn_ref, oracle.tree_attn_dense_ref])
def test_zero_queries_average_the_hand_derived_visible_rows(attn):
    assert pins.pin_golden_uniform(attn, np.random.default_rng(13)) < TIGHT


def all_parent_arrays(n):
    return itertools.product(*[range(-1, i) for i in range(n)])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_bruteforce_all_small_trees_two_formulations_agree(n):
    """Every parent array with parent[i] in {-1..i-1}: n! of them (720 at n = 6)."""
    rng = np.random.default_rng(100 + n)
    P, hq, hkv, d = 3, 2, 1, 4
    count = 0
    for parent in all_parent_arrays(n):
        parent = list(parent)
        cap = P + n
        q = rng.standard_normal((n, hq, d))
        k = rng.standard_normal((hkv, cap, d))
        v = rng.standard_normal((hkv, cap, d))
        a = oracle.tree_attn_ref(q, k, v, P, parent, hkv)
        b = oracle.tree_attn_dense_ref(q, k, v, P, parent, hkv)
        assert np.abs(a - b).max() < TIGHT, parent
        count += 1
    assert count == np.prod(range(1, n + 1))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_bruteforce_every_node_of_every_small_tree_is_causal_after_reroot(n):
    rng = np.random.default_rng(200 + n)
    for parent in all_parent_arrays(n):
        parent = list(parent)
        for x in range(n):
            err = pins.pin_path_reroot_causal(oracle.tree_attn_ref, oracle.kv_reroot_ref,
                                              parent, x, rng)
            assert err < TIGHT, (parent, x)


@pytest.mark.parametrize("attn", [oracle.tree_attn_ref, oracle.tree_attn_dense_ref])
@pytest.mark.parametrize("shape", [(29, 12, 4, 4, 2, 8), (0, 8, 8, 2, 1, 16), (5, 3, 1, 2, 2, 4)])
def test_chain_frontier_queries_are_causal_attention(attn, shape):
    P, n, w, hq, hkv, d = shape
    assert pins.pin_chain_frontier_causal(attn, np.random.default_rng(15), P, n, w, hq, hkv, d) < TIGHT


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_bruteforce_frontier_rows_do_not_depend_on_other_queries(n):
    """For every small tree and every q_first: both formulations give the
    full tree's rows from q_first on, whatever the earlier nodes' queries are."""
    rng = np.random.default_rng(300 + n)
    P, hq, hkv, d = 2, 2, 1, 4
    for parent in all_parent_arrays(n):
        parent = list(parent)
        k = rng.standard_normal((hkv, P + n, d))
        v = rng.standard_normal((hkv, P + n, d))
        q = rng.standard_normal((n, hq, d))
        full = oracle.tree_attn_dense_ref(q, k, v, P, parent, hkv)
        for qf in range(n + 1):
            q2 = q.copy()
            q2[:qf] = rng.standard_normal((qf, hq, d))  # the other nodes' queries change
            for attn in (oracle.tree_attn_ref, oracle.tree_attn_dense_ref):
                got = attn(q2[qf:], k, v, P, parent, hkv, q_first=qf)
                assert got.shape == (n - qf, hq, d)
                if n - qf:
                    assert np.abs(got - full[qf:]).max() < TIGHT, (parent, qf)


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(14)
    P, n, hq, hkv, d = 20, 12, 6, 3, 8
    parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
    c = rng.standard_normal(d)
    k = rng.standard_normal((hkv, P + n, d)) * 3
    v = np.broadcast_to(c, (hkv, P + n, d)).copy()
    q = rng.standard_normal((n, hq, d)) * 3
    for attn in (oracle.tree_attn_ref, oracle.tree_attn_dense_ref):
        out = attn(q, k, v, P, parent, hkv)
        assert np.abs(out - c).max() < 1e-13


def test_one_hot_values_expose_weights_and_exact_zeros():
    """V row t = e_t turns the output into the attention weights themselves."""
    rng = np.random.default_rng(15)
    P, n, hq, hkv = 10, 7, 2, 1
    d = P + n
    parent = [-1, 0, 0, 1, -1, 4, 3]
    k = rng.standard_normal((hkv, P + n, d))
    v = np.eye(P + n)[None]
    q = rng.standard_normal((n, hq, d))
    gold = pins.load_golden("mask_visible_sets.json")["cases"][0]
    assert gold["parent"] == parent
    for attn in (oracle.tree_attn_ref, oracle.tree_attn_dense_ref):
        w = attn(q, k, v, P, parent, hkv)
        assert np.abs(w.sum(axis=-1) - 1).max() < 1e-13
        for i, vis in enumerate(gold["visible"]):
            hidden = [P + j for j in range(n) if j not in vis]
            seen = list(range(P)) + [P + j for j in vis]
            assert (w[i, :, hidden] == 0.0).all()
            assert (w[i, :, seen] > 0.0).all()


def test_topological_relabelling_permutes_outputs():
    rng = np.random.default_rng(16)
    P, n, hq, hkv, d = 9, 12, 4, 2, 8
    parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
    # A random topological order: repeatedly pick a random node whose parent is placed.
    placed, order = set(), []
    while len(order) < n:
        ready = [i for i in range(n) if i not in placed and (parent[i] == -1 or parent[i] in placed)]
        pick = ready[int(rng.integers(0, len(ready)))]
        order.append(pick)
        placed.add(pick)
    new_of = {old: new for new, old in enumerate(order)}
    parent2 = [-1 if parent[o] == -1 else new_of[parent[o]] for o in order]
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((hkv, P + n, d))
    v = rng.standard_normal((hkv, P + n, d))
    k2, v2 = k.copy(), v.copy()
    k2[:, P:] = k[:, [P + o for o in order]]
    v2[:, P:] = v[:, [P + o for o in order]]
    a = oracle.tree_attn_ref(q, k, v, P, parent, hkv)
    b = oracle.tree_attn_ref(q[order], k2, v2, P, parent2, hkv)
    assert np.abs(a[order] - b).max() < TIGHT


def test_slots_beyond_the_tree_are_never_read():
    rng = np.random.default_rng(17)
    P, n, hq, hkv, d = 5, 6, 2, 1, 4
    parent = [-1, 0, 1, -1, 3, 0]
    k = rng.standard_normal((hkv, P + n + 4, d))
    v = rng.standard_normal((hkv, P + n + 4, d))
    q = rng.standard_normal((n, hq, d))
    for attn in (oracle.tree_attn_ref, oracle.tree_attn_dense_ref):
        clean = attn(q, k, v, P, parent, hkv)
        kp, vp = k.copy(), v.copy()
        kp[:, P + n:] = np.nan
        vp[:, P + n:] = np.nan
        assert np.array_equal(attn(q, kp, vp, P, parent, hkv), clean)


def test_bad_parent_arrays_are_rejected():
    for bad in ([0], [-1, 1], [-1, 0, 3], [-2]):
        with pytest.raises(ValueError):
            oracle.check_parent(bad)


# ----------------------------------------------------------------------------- re-root

def test_reroot_hand_worked_cases():
    assert pins.pin_reroot_golden(oracle.reroot_plan_ref) == 0


def test_reroot_invalid_requests_are_rejected():
    for case in pins.load_golden("reroot_cases.json")["invalid"]:
        cap = case["prefix_len"] + len(case["parent"])
        with pytest.raises(ValueError):
            oracle.reroot_plan_ref(case["prefix_len"], case["parent"], case["path"],
                                   case["survivors"], cap)


def test_reroot_rejects_capacity_overflow():
    with pytest.raises(ValueError):
        oracle.reroot_plan_ref(10, [-1, 0], [0], [1], 11)


@st.composite
def reroot_requests(draw):
    n = draw(st.integers(1, 12))
    parent = [draw(st.integers(-1, i - 1)) for i in range(n)]
    roots = [i for i in range(n) if parent[i] == -1]
    kids = [[j for j in range(n) if parent[j] == i] for i in range(n)]
    m_max = draw(st.integers(0, n))
    path = []
    if m_max and roots:
        path = [draw(st.sampled_from(roots))]
        while len(path) < m_max and kids[path[-1]]:
            path.append(draw(st.sampled_from(kids[path[-1]])))
    last = path[-1] if path else -1
    # survivors: a random parent-closed subset of last's strict descendants
    cand = [j for j in range(n) if j not in path]
    surv = []
    for j in sorted(cand):
        if (parent[j] == last or parent[j] in surv) and draw(st.booleans()):
            surv.append(j)
    P = draw(st.integers(0, 6))
    return P, parent, path, surv


@settings(max_examples=150, deadline=None)
@given(reroot_requests(), st.integers(0, 2**31 - 1))
def test_reroot_bytes_and_attention_invariant(req, seed):
    """Byte layout of the gather, plus: re-rooting and then attending gives every
    survivor the output it had on the original cache, and every accepted node
    the causal-attention output at its new prefix position."""
    P, parent, path, surv = req
    rng = np.random.default_rng(seed)
    n, hq, hkv, d, L = len(parent), 4, 2, 8, 2
    cap = P + n + 3
    k = rng.standard_normal((L, hkv, cap, d))
    v = rng.standard_normal((L, hkv, cap, d))
    k2, v2, new_p, new_par = oracle.kv_reroot_ref(k, v, P, parent, path, surv)
    order = path + surv
    end = P + len(order)
    assert new_p == P + len(path)
    assert np.array_equal(k2[:, :, :P], k[:, :, :P]) and np.array_equal(k2[:, :, end:], k[:, :, end:])
    assert np.array_equal(v2[:, :, :P], v[:, :, :P]) and np.array_equal(v2[:, :, end:], v[:, :, end:])
    for j, o in enumerate(order):
        assert np.array_equal(k2[:, :, P + j], k[:, :, P + o])
        assert np.array_equal(v2[:, :, P + j], v[:, :, P + o])
    for kk, s in enumerate(surv):
        assert new_par[kk] < kk
        assert (new_par[kk] == -1) == (parent[s] == (path[-1] if path else -1))
        if new_par[kk] >= 0:
            assert surv[new_par[kk]] == parent[s]

    q = rng.standard_normal((n, hq, d))
    before = oracle.tree_attn_ref(q, k[1], v[1], P, parent, hkv)
    if surv:
        after = oracle.tree_attn_ref(q[surv], k2[1], v2[1], new_p, new_par, hkv)
        assert np.abs(after - before[surv]).max() < TIGHT
    if path:
        q_seq = np.zeros((new_p, hq, d))
        q_seq[P:] = q[path]
        causal = pins.sdpa_causal(q_seq, k2[1, :, :new_p].transpose(1, 0, 2).copy(),
                                  v2[1, :, :new_p].transpose(1, 0, 2).copy())
        assert np.abs(causal[P:] - before[path]).max() < TIGHT


def test_reroot_works_on_raw_bf16_words():
    rng = np.random.default_rng(18)
    k = rng.integers(0, 2**16, size=(2, 3, 20, 8), dtype=np.uint16)
    v = rng.integers(0, 2**16, size=(2, 3, 20, 8), dtype=np.uint16)
    k2, v2, new_p, new_par = oracle.kv_reroot_ref(k, v, 4, [-1, 0, 0, 1, 1], [0, 1], [3, 4])
    assert k2.dtype == np.uint16 and new_p == 6 and new_par == [-1, -1]
    assert np.array_equal(k2[:, :, 6], k[:, :, 7]) and np.array_equal(k2[:, :, 7], k[:, :, 8])
    assert np.array_equal(k2[:, :, 8:], k[:, :, 8:])


# ---------------------------------------------------------------------------
# Tree verification

def test_verify_hand_worked_cases():
    assert pins.pin_verify_golden(oracle.tree_verify_ref) == 0


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_verify_bruteforce_all_small_trees_match_the_top_down_walk(n):
    rng = np.random.default_rng(100 + n)
    parents = [list(p) for p in all_parent_arrays(n)]
    assert pins.pin_verify_walk(oracle.tree_verify_ref, parents, rng) == 0


def test_verify_random_larger_trees_match_the_top_down_walk():
    rng = np.random.default_rng(7)
    parents = [[-1] + [int(rng.integers(-1, i)) for i in range(1, n)] for n in (16, 33, 64) for _ in range(20)]
    assert pins.pin_verify_walk(oracle.tree_verify_ref, parents, rng, vocab=4, draws=2) == 0


def test_verify_chain_accepts_exactly_the_agreeing_prefix():
    assert pins.pin_verify_chain(oracle.tree_verify_ref, np.random.default_rng(8)) == 0


def test_row_argmax_is_the_first_maximum_and_ignores_the_sign_of_zero():
    x = np.array([[1, 3, 3, 0], [-np.inf] * 4, [-0.0, 0.0, -1, 0.0], [2, 1, 2, np.inf]], dtype=np.float32)
    assert list(oracle.row_argmax(x)) == [1, 0, 0, 3]
    bf = np.array([[0x3F80, 0x4000, 0x4000]], dtype=np.uint16)  # bf16 words 1, 2, 2
    assert list(oracle.row_argmax((bf.astype(np.uint32) << 16).view(np.float32))) == [1]


def test_verify_rejects_malformed_inputs():
    with pytest.raises(ValueError):
        oracle.tree_verify_ref(np.zeros((2, 4)), [0, 0], [-1, 0])  # one row short
    with pytest.raises(ValueError):
        oracle.tree_verify_ref(np.zeros((3, 4)), [0], [-1, 0])  # one token short
    with pytest.raises(ValueError):
        oracle.tree_verify_ref(np.zeros((3, 4)), [0, 0], [-1, 1])  # parent not before the node


# ---------------------------------------------------------------------------
# Maximum-likelihood expansion

def test_expand_hand_worked_cases():
    assert pins.pin_expand_golden(oracle.tree_expand_ref) < 1e-12


def test_expand_matches_global_bruteforce_with_library_log_softmax():
    assert pins.pin_expand_bruteforce(oracle.tree_expand_ref, np.random.default_rng(31)) < 1e-12


def test_expand_uniform_rows_closed_form():
    assert pins.pin_expand_uniform(oracle.tree_expand_ref, np.random.default_rng(32)) < 1e-12


def test_log_softmax_rows_normalises_and_matches_the_library():
    from scipy.special import log_softmax
    rng = np.random.default_rng(33)
    x = rng.standard_normal((5, 1000)) * 20 + np.array([[0], [500], [-500], [1e4], [3]])
    got = oracle.log_softmax_rows(x)
    assert np.abs(got - log_softmax(x, axis=1)).max() < 1e-9
    assert np.abs(np.exp(got).sum(axis=1) - 1).max() < 1e-12


def test_expand_rejects_malformed_inputs():
    with pytest.raises(ValueError):
        oracle.tree_expand_ref(np.zeros((2, 3)), [0.0], 1)
    with pytest.raises(ValueError):
        oracle.tree_expand_ref(np.zeros((2, 3)), [0.0, 0.0], 7)
    with pytest.raises(ValueError):
        oracle.tree_expand_ref(np.full((1, 3), -np.inf), [0.0], 1)
