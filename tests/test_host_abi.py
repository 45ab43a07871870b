"""The C-ABI library on the CPU: exports, host planning, validation errors.

No test here launches a kernel: every call either runs host-only code or fails
validation before anything would be enqueued (fake device addresses below are
never dereferenced).
"""

import ctypes
import os
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings

import oracle
import tree_masked_attention_attn_amd as ta
from tests import pins
from tests.test_oracle_pins import reroot_requests

FAKE = 1 << 40  # 16-byte aligned, never dereferenced


def test_library_exports_every_declared_symbol():
    names = ta.header_symbols()
    assert len(names) >= 9
    lib = ta.lib()
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ta.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    assert ta.lib().ta_abi_version() == 1


def test_status_strings():
    for s in range(6):
        assert ta.lib().ta_status_string(s)


def test_ancestor_bits_match_oracle_walk():
    rng = np.random.default_rng(0)
    trees = [c["parent"] for c in pins.load_golden("mask_visible_sets.json")["cases"]]
    trees += [[-1] + [int(rng.integers(-1, i)) for i in range(1, n)] for n in (1, 2, 17, 63, 64, 65, 100, 128)]
    trees += [[-1] + list(range(127)), [-1] * 128]
    for parent in trees:
        bits = ta.tree_ancestor_bits(parent)
        for i, b in enumerate(bits):
            assert [j for j in range(128) if (b >> j) & 1] == oracle.ancestors_inclusive(parent, i)


def test_one_word_ancestor_bits_match_the_two_word_sets_up_to_64_nodes():
    rng = np.random.default_rng(1)
    for n in (1, 9, 64):
        parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
        par, _ = ta._i32(parent)
        one = (ctypes.c_uint64 * n)()
        assert ta.lib().ta_tree_ancestor_bits(par, n, one) == ta.TA_OK
        assert list(one) == ta.tree_ancestor_bits(parent)
    par, _ = ta._i32([-1] * 65)
    assert ta.lib().ta_tree_ancestor_bits(par, 65, (ctypes.c_uint64 * 65)()) == ta.TA_ERR_UNSUPPORTED


def test_ancestor_bits_reject_bad_trees():
    for bad, status in (([0], ta.TA_ERR_TREE), ([-1, 1], ta.TA_ERR_TREE), ([-1, 0, 5], ta.TA_ERR_TREE),
                        ([-1] * 129, ta.TA_ERR_UNSUPPORTED)):
        with pytest.raises(ta.TreeAttnError) as e:
            ta.tree_ancestor_bits(bad)
        assert e.value.status == status


def test_reroot_plan_hand_worked_cases():
    def plan(P, parent, path, surv, cap):
        src, new_par, new_p = ta.kv_reroot_plan(P, cap, parent, path, surv)
        return [s - P for s in src], new_p, new_par
    assert pins.pin_reroot_golden(plan) == 0


def test_reroot_plan_rejects_invalid_requests():
    for case in pins.load_golden("reroot_cases.json")["invalid"]:
        cap = case["prefix_len"] + len(case["parent"])
        with pytest.raises(ta.TreeAttnError) as e:
            ta.kv_reroot_plan(case["prefix_len"], cap, case["parent"], case["path"], case["survivors"])
        assert e.value.status == ta.TA_ERR_TREE, case["name"]
    with pytest.raises(ta.TreeAttnError) as e:
        ta.kv_reroot_plan(10, 11, [-1, 0], [0], [1])
    assert e.value.status == ta.TA_ERR_CAPACITY


@settings(max_examples=300, deadline=None)
@given(reroot_requests())
def test_reroot_plan_matches_oracle(req):
    P, parent, path, surv = req
    cap = P + len(parent) + 1
    order, new_p, new_par = oracle.reroot_plan_ref(P, parent, path, surv, cap)
    src, new_par2, new_p2 = ta.kv_reroot_plan(P, cap, parent, path, surv)
    assert src == [P + o for o in order] and new_par2 == new_par and new_p2 == new_p
    # the properties the in-place copy relies on
    assert all(s >= P + k for k, s in enumerate(src))
    assert all(b > a for a, b in zip(src, src[1:]))


def _desc(L=1, H=8, C=8448, D=128, dtype=ta.TA_BF16, k=FAKE, v=FAKE + (1 << 30)):
    return ta.ta_kv_cache(k, v, L, H, C, D, dtype)


def _attn(desc, n_q_heads=64, prefix=8192, parent=None, q=FAKE, out=FAKE, ws=None, ws_len=0, layer=0):
    parent = [-1] * 8 if parent is None else parent
    par, n = ta._i32(parent)
    return ta.lib().ta_tree_attn(q, ctypes.byref(desc), layer, prefix, par, n, n_q_heads, out, ws, ws_len, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(desc=_desc(D=96)), ta.TA_ERR_UNSUPPORTED),
    (dict(desc=_desc(dtype=7)), ta.TA_ERR_UNSUPPORTED),
    (dict(desc=_desc(), n_q_heads=60), ta.TA_ERR_UNSUPPORTED),
    (dict(desc=_desc(H=2), n_q_heads=64), ta.TA_ERR_UNSUPPORTED),   # 32 q heads per KV head
    (dict(desc=_desc(), parent=[-1] * 129), ta.TA_ERR_UNSUPPORTED),
    (dict(desc=_desc(), prefix=8448 - 7), ta.TA_ERR_CAPACITY),
    (dict(desc=_desc(), prefix=-1), ta.TA_ERR_ARG),
    (dict(desc=_desc(), parent=[-1, 1]), ta.TA_ERR_TREE),
    (dict(desc=_desc(k=FAKE + 8)), ta.TA_ERR_ARG),
    (dict(desc=_desc(k=0)), ta.TA_ERR_ARG),
    (dict(desc=_desc(), q=FAKE + 4), ta.TA_ERR_ARG),
    (dict(desc=_desc(), out=0), ta.TA_ERR_ARG),
    (dict(desc=_desc(), layer=1), ta.TA_ERR_ARG),
    (dict(desc=_desc(L=0)), ta.TA_ERR_ARG),
    (dict(desc=_desc()), ta.TA_ERR_ARG),                 # needs a workspace, none given
    (dict(desc=_desc(), ws=FAKE, ws_len=1024), ta.TA_ERR_ARG),
])
def test_tree_attn_rejects_before_enqueueing(kwargs, status):
    assert _attn(**kwargs) == status
    assert ta.lib().ta_last_error()


def test_empty_tree_is_a_no_op():
    assert _attn(_desc(), parent=[]) == ta.TA_OK


def test_frontier_rows_validation():
    d = _desc()
    par, n = ta._i32([-1] * 8)

    def rows(q_first, ws=None, ws_len=0):
        return ta.lib().ta_tree_attn_rows(FAKE, ctypes.byref(d), 0, 8192, par, n, q_first, 64, FAKE, ws, ws_len,
                                          None)
    assert rows(-1) == ta.TA_ERR_ARG and rows(9) == ta.TA_ERR_ARG
    assert rows(8) == ta.TA_OK  # no query rows: nothing is enqueued
    assert rows(4) == ta.TA_ERR_ARG  # needs a workspace
    lib = ta.lib()
    full = lib.ta_tree_attn_rows_workspace_bytes(ctypes.byref(d), 64, 8192, 8, 0)
    assert full == lib.ta_tree_attn_workspace_bytes(ctypes.byref(d), 64, 8192, 8)
    assert lib.ta_tree_attn_rows_workspace_bytes(ctypes.byref(d), 64, 8192, 8, 9) == 0
    assert lib.ta_tree_attn_rows_num_splits(ctypes.byref(d), 64, 8192, 8, 4) >= 1


def test_workspace_and_split_plan():
    lib = ta.lib()
    d = _desc()
    assert lib.ta_tree_attn_num_splits(ctypes.byref(d), 64, 8192, 64) > 1
    ws = lib.ta_tree_attn_workspace_bytes(ctypes.byref(d), 64, 8192, 64)
    assert ws > 0 and ws % 256 == 0
    tiny = _desc(H=1, C=256, D=64, dtype=ta.TA_F32)
    assert lib.ta_tree_attn_num_splits(ctypes.byref(tiny), 2, 128, 15) == 1
    assert lib.ta_tree_attn_workspace_bytes(ctypes.byref(tiny), 2, 128, 15) == 0
    assert lib.ta_tree_attn_workspace_bytes(ctypes.byref(d), 60, 8192, 64) == 0  # invalid -> 0
    assert lib.ta_tree_attn_rows_block_rows(ctypes.byref(d), 60, 8192, 64, 0) == 0
    assert lib.ta_tree_attn_rows_block_rows(ctypes.byref(d), 64, 8192, 8, 0) == 64   # 64 rows per KV head
    assert lib.ta_tree_attn_rows_block_rows(ctypes.byref(tiny), 2, 128, 15, 0) == 128  # fp32


def _units_from_workspace(ws, head_dim):
    """Work units (workgroups) of a split launch, read back from its workspace
    size: 4096 x 16 B of counters, then (max, sum) and partial-output rows
    for 128 rows per unit, each part 256-byte aligned."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    size = lambda u: up(up(4096 * 16 + u * 128 * 8) + u * 128 * head_dim * 4)  # noqa: E731
    units = [u for u in range(1, 1 << 17) if size(u) == ws]
    assert len(units) == 1
    return units[0]


@pytest.mark.parametrize("name,n_kv,group,prefix,n_tree,dtype,block", [
    ("8B verify: 128-row blocks fill only 128 units", 8, 4, 2048, 64, ta.TA_BF16, 64),
    ("70B verify, TP = 4 share", 2, 8, 8192, 64, ta.TA_BF16, 64),
    ("ragged: 300 rows per KV head", 4, 3, 1000, 100, ta.TA_BF16, 64),
    ("70B verify: 256 units at 128 rows already", 8, 8, 8192, 64, ta.TA_BF16, 128),
    ("draft loop: 256 units either way, 64-row splits of 9 stages", 8, 4, 4096, 64, ta.TA_BF16, 64),
    ("70B heads, P = 2048: 256 units either way, 9 stages", 8, 8, 2048, 64, ta.TA_BF16, 64),
    ("70B heads, P = 4096: 256 units either way, 17 stages", 8, 8, 4096, 64, ta.TA_BF16, 128),
    ("fp32 keeps 128-row blocks", 2, 8, 8192, 64, ta.TA_F32, 128),
    ("64-row blocks would give 280 units (last block 32 rows)", 8, 8, 2000, 36, ta.TA_BF16, 128),
    ("256 units either way, 64-row splits of 16 stages (last block 96 rows)", 8, 8, 4000, 60, ta.TA_BF16, 128),
])
def test_row_block_choice(name, n_kv, group, prefix, n_tree, dtype, block):
    """bf16 launches whose 128-row blocks leave CUs idle (fewer than 256
    workgroups once the splits are capped at 4 stages each) take 64-row
    blocks instead, and so do launches where both give 256 units and the
    64-row splits carry at most 12 stages; the unit count read back from the
    workspace size is KV heads x row blocks x splits for the block size
    chosen."""
    lib = ta.lib()
    d = _desc(H=n_kv, C=prefix + n_tree, dtype=dtype)
    splits = lib.ta_tree_attn_num_splits(ctypes.byref(d), n_kv * group, prefix, n_tree)
    ws = lib.ta_tree_attn_workspace_bytes(ctypes.byref(d), n_kv * group, prefix, n_tree)
    assert splits > 1 and ws > 0
    assert lib.ta_tree_attn_rows_block_rows(ctypes.byref(d), n_kv * group, prefix, n_tree, 0) == block
    blocks = -(-group * n_tree // block)
    assert _units_from_workspace(ws, 128) == n_kv * blocks * splits, name
    assert n_kv * blocks * splits <= 256


def test_kv_reroot_rejects_before_enqueueing():
    lib = ta.lib()
    np_out = (ctypes.c_int32 * 128)()
    npl = ctypes.c_int32(-7)

    def call(desc, P, parent, path, surv, new_parent=np_out, new_prefix=ctypes.byref(npl)):
        par, n = ta._i32(parent)
        a, m = ta._i32(path)
        s, k = ta._i32(surv)
        return lib.ta_kv_reroot(ctypes.byref(desc), P, par, n, a, m, s, k, new_parent, new_prefix, None)

    d = _desc(C=100)
    assert call(d, 0, [-1, 0, 0, 1], [0, 2, 3], []) == ta.TA_ERR_TREE
    assert call(d, 0, [-1, 0, 0, 1], [0, 1], [2]) == ta.TA_ERR_TREE
    assert call(d, 99, [-1, 0], [0], [1]) == ta.TA_ERR_CAPACITY
    assert call(_desc(D=80), 0, [-1], [0], []) == ta.TA_ERR_UNSUPPORTED
    assert call(_desc(v=0), 0, [-1], [0], []) == ta.TA_ERR_ARG
    assert call(d, 0, [-1, 0], [0], [1], new_prefix=None) == ta.TA_ERR_ARG
    assert npl.value == -7  # outputs untouched on error
    # A valid request whose rows are already in place moves nothing: host-only.
    assert call(d, 5, [-1, 0, 1], [0, 1], [2]) == ta.TA_OK
    assert npl.value == 7 and np_out[0] == -1


def test_package_refuses_to_run_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ta, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ta, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        ta.tree_ancestor_bits([-1])


def test_package_does_not_import_the_oracle():
    pkg = os.path.dirname(ta.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text


def _verify_call(logits=FAKE, dtype=ta.TA_BF16, vocab=1000, stride=1000, tokens=FAKE, parent=(-1, 0),
                 choice=FAKE, result=FAKE, ws=FAKE, ws_len=16384):
    par, n = ta._i32(parent)
    return ta.lib().ta_tree_verify(logits, dtype, vocab, stride, tokens, par, n, choice, result, ws, ws_len, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(dtype=7), ta.TA_ERR_UNSUPPORTED),
    (dict(vocab=0, stride=8), ta.TA_ERR_ARG),
    (dict(vocab=1 << 31, stride=1 << 31), ta.TA_ERR_ARG),
    (dict(stride=999), ta.TA_ERR_ARG),
    (dict(vocab=1001, stride=1001), ta.TA_ERR_ARG),  # rows not 16-byte aligned in bf16
    (dict(dtype=ta.TA_F32, vocab=1002, stride=1002), ta.TA_ERR_ARG),
    (dict(logits=None), ta.TA_ERR_ARG),
    (dict(tokens=None), ta.TA_ERR_ARG),
    (dict(choice=None), ta.TA_ERR_ARG),
    (dict(result=None), ta.TA_ERR_ARG),
    (dict(logits=FAKE + 8), ta.TA_ERR_ARG),
    (dict(result=FAKE + 2), ta.TA_ERR_ARG),
    (dict(ws=None), ta.TA_ERR_ARG),
    (dict(ws_len=16), ta.TA_ERR_ARG),
    (dict(ws=FAKE + 16), ta.TA_ERR_ARG),
    (dict(parent=(0,)), ta.TA_ERR_TREE),
    (dict(parent=(-1,) * 129), ta.TA_ERR_UNSUPPORTED),
])
def test_tree_verify_rejects_before_enqueueing(kwargs, status):
    assert _verify_call(**kwargs) == status
    assert ta.lib().ta_last_error()


def test_tree_verify_workspace_bytes():
    L = ta.lib()
    sizes = {L.ta_tree_verify_workspace_bytes(n) for n in range(129)}
    assert len(sizes) == 1 and 0 < sizes.pop() <= 16384
    assert L.ta_tree_verify_workspace_bytes(129) == 0 and L.ta_tree_verify_workspace_bytes(-1) == 0


def _expand_call(logits=FAKE, dtype=ta.TA_BF16, vocab=1000, stride=1000, scores=FAKE, w=8, k=8,
                 leaf=FAKE, token=FAKE, score=FAKE, ws=FAKE, ws_len=1 << 21):
    return ta.lib().ta_tree_expand(logits, dtype, vocab, stride, scores, w, k, leaf, token, score, ws, ws_len, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(dtype=5), ta.TA_ERR_UNSUPPORTED),
    (dict(w=0), ta.TA_ERR_UNSUPPORTED),
    (dict(w=65), ta.TA_ERR_UNSUPPORTED),
    (dict(k=0), ta.TA_ERR_UNSUPPORTED),
    (dict(k=17), ta.TA_ERR_UNSUPPORTED),
    (dict(vocab=0, stride=8), ta.TA_ERR_UNSUPPORTED),
    (dict(vocab=262145, stride=262152), ta.TA_ERR_UNSUPPORTED),
    (dict(vocab=1, stride=8, w=2, k=3), ta.TA_ERR_ARG),  # k > w * vocab
    (dict(stride=999), ta.TA_ERR_ARG),
    (dict(vocab=1001, stride=1001), ta.TA_ERR_ARG),
    (dict(logits=None), ta.TA_ERR_ARG),
    (dict(scores=None), ta.TA_ERR_ARG),
    (dict(score=None), ta.TA_ERR_ARG),
    (dict(logits=FAKE + 4), ta.TA_ERR_ARG),
    (dict(token=FAKE + 1), ta.TA_ERR_ARG),
    (dict(ws=None), ta.TA_ERR_ARG),
    (dict(ws_len=1024), ta.TA_ERR_ARG),
    (dict(ws=FAKE + 64), ta.TA_ERR_ARG),
])
def test_tree_expand_rejects_before_enqueueing(kwargs, status):
    assert _expand_call(**kwargs) == status
    assert ta.lib().ta_last_error()


def test_tree_expand_workspace_bytes():
    L = ta.lib()
    assert L.ta_tree_expand_workspace_bytes(0) == 0 and L.ta_tree_expand_workspace_bytes(65) == 0
    sizes = [L.ta_tree_expand_workspace_bytes(w) for w in range(1, 65)]
    assert all(b > a for a, b in zip(sizes, sizes[1:])) and sizes[-1] <= 2 << 20


def test_shapes_past_the_kernels_32_bit_ranges_are_refused():
    """A KV head's [prefix | tree] bytes and one call's query bytes are
    addressed through 32-bit buffer ranges, and work-unit ids are divided
    exactly only below 2^17: such shapes fail validation before anything is
    enqueued instead of being mis-addressed."""
    lib = ta.lib()
    par, n = ta._i32([-1] * 8)
    keys_ok = (2 ** 31 - 1 - 2 ** 20) // 256 - 8  # bf16, head_dim 128: 256 bytes per key
    big = _desc(H=1, C=keys_ok + 64)
    assert lib.ta_tree_attn_rows(FAKE, ctypes.byref(big), 0, keys_ok + 1, par, n, 0, 4, FAKE, None, 0,
                                 None) == ta.TA_ERR_UNSUPPORTED
    assert b"32-bit" in lib.ta_last_error()
    assert lib.ta_tree_attn_workspace_bytes(ctypes.byref(big), 4, keys_ok, n) > 0  # at the bound: planned
    f32 = _desc(H=1, C=keys_ok + 64, dtype=ta.TA_F32)  # 512 bytes per key: half as many keys
    assert lib.ta_tree_attn_workspace_bytes(ctypes.byref(f32), 4, keys_ok // 2 + 1, n) == 0
    # 140000 KV heads of one query row each: one unit per head and no split
    many = _desc(H=140000, C=64, D=64)
    one, _ = ta._i32([-1])
    assert lib.ta_tree_attn_rows(FAKE, ctypes.byref(many), 0, 8, one, 1, 0, 140000, FAKE, None, 0,
                                 None) == ta.TA_ERR_UNSUPPORTED
    assert b"work units" in lib.ta_last_error()
    fewer = _desc(H=120000, C=64, D=64)
    assert lib.ta_tree_attn_num_splits(ctypes.byref(fewer), 120000, 8, 1) == 1


def test_default_workspaces_are_kept_per_stream():
    """Two streams of one device must not share the split counters and
    partial rows of one workspace; calls on one stream reuse theirs."""
    a = ta._workspace("cpu", 4096, "attn", stream=11)
    b = ta._workspace("cpu", 4096, "attn", stream=12)
    assert a.data_ptr() != b.data_ptr()
    assert ta._workspace("cpu", 4096, "attn", stream=11).data_ptr() == a.data_ptr()
    assert ta._workspace("cpu", 4096, "verify", stream=11).data_ptr() != a.data_ptr()
    grown = ta._workspace("cpu", 8 << 20, "attn", stream=11)
    assert grown.numel() >= 8 << 20 and ta._workspace("cpu", 16, "attn", stream=11).data_ptr() == grown.data_ptr()
    assert ta._workspace("cpu", 0, "attn", stream=11) is None


def test_noalloc_entry_refuses_shapes_beyond_its_scratch_before_any_device_call():
    """255 KV heads of 64 query rows each at 2 splits: 510 units of fp32
    partials (33 MB) exceed the 20 MiB static scratch."""
    lib = ta.lib()
    d = _desc(H=255, C=1200)
    par, n = ta._i32([-1] * 64)
    need = lib.ta_tree_attn_rows_workspace_bytes(ctypes.byref(d), 255, 1000, 64, 0)
    assert need > 20 << 20
    st = lib.ta_tree_attn_rows_noalloc(FAKE, ctypes.byref(d), 0, 1000, par, n, 0, 255, FAKE, None)
    assert st == ta.TA_ERR_UNSUPPORTED and b"static scratch" in lib.ta_last_error()
    bad, _ = ta._i32([-1, 5] + [0] * 62)
    assert lib.ta_tree_attn_rows_noalloc(FAKE, ctypes.byref(_desc()), 0, 8192, bad, 64, 0, 64, FAKE,
                                         None) == ta.TA_ERR_TREE
