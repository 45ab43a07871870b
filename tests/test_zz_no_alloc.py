"""The allocation-free entry point on the GPU: ta_tree_attn_rows_noalloc,
called through the C ABI, against ta_tree_attn_rows with its own workspace,
on two calls in a row (the second a smaller input), then the same against the
oracle. Both run the same kernels and plan, so the outputs must be bitwise
identical; the oracle check holds them to the bf16 bar."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_attn_amd as ta
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def noalloc(x, cfg, out):
    q, k, v = x["q"], x["k"], x["v"]
    desc = ta._cache_desc(k, v)
    par, n = ta._i32(x["parent"])
    st = ta.lib().ta_tree_attn_rows_noalloc(q.data_ptr(), ctypes.byref(desc), 0, x["prefix_len"], par, n,
                                            x.get("q_first", 0), cfg["n_q_heads"], out.data_ptr(),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    ta._check(st)
    return out


@pytest.mark.parametrize("names", [("llama3_70b_verify", "llama3_8b_verify"),
                                   ("llama3_8b_verify", "draft_expand_w8")])
def test_noalloc_matches_the_workspace_entry_point(names):
    for name in names:
        cfg = W.config(name)
        x = W.make_inputs(cfg)
        g = {key: x[key].to(DEV) for key in ("q", "k", "v")}
        g.update(prefix_len=x["prefix_len"], parent=x["parent"], q_first=x["q_first"])
        splits = ta.tree_attn_num_splits(g["k"], g["v"], cfg["n_q_heads"], x["prefix_len"], cfg["n_tree"],
                                          x["q_first"])
        print(f"[no-alloc] {name} splits={splits}", file=sys.stderr, flush=True)
        assert splits > 1  # the scratch carries split partials and counters
        got = noalloc(g, cfg, torch.full_like(g["q"], float("nan")))
        want = ta.tree_attn(g["q"], g["k"], g["v"], x["prefix_len"], x["parent"], q_first=x["q_first"])
        torch.cuda.synchronize()
        assert torch.equal(got, want), name
        ref = oracle.tree_attn_dense_ref(W.to_f64(x["q"]), W.to_f64(x["k"][0]), W.to_f64(x["v"][0]),
                                         x["prefix_len"], x["parent"], cfg["n_kv_heads"], q_first=x["q_first"])
        err = float(np.abs(W.to_f64(got) - ref).max())
        assert err <= 1e-2 and err <= 2.0 ** -7 * float(np.abs(ref).max()) + 1e-6, (name, err)
