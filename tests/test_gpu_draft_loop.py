"""The draft-loop workload end to end on the GPU: 100 iterations of tree
attention over a 64-node tree, an accepted path of length 1..8, re-root of the
surviving subtree and refill. Every iteration's attention is checked against the
oracle, every re-root's host outputs must match, and the final cache must be
byte-identical to the oracle's cache after the same 100 steps."""

import sys

import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_attn_amd as ta
import workloads as W
from tests.test_gpu_parity import check_close

pytestmark = pytest.mark.gpu


def test_draft_loop_100_iterations():
    cfg = W.config("draft_loop_1b")
    loop = W.DraftLoop(cfg)
    k, v = loop.initial_cache()
    end = loop.prefix_len + cfg["n_tree"]
    k[:, :, end:] = float("nan")
    v[:, :, end:] = float("nan")
    kd, vd = k.cuda(), v.cuda()
    kb, vb = W.raw_bits(k), W.raw_bits(v)
    hkv = cfg["n_kv_heads"]
    worst = 0.0
    for it in range(cfg["iterations"]):
        q = loop.queries()
        P, parent = loop.prefix_len, list(loop.parent)
        out = ta.tree_attn(q.cuda(), kd, vd, P, parent)
        path, surv = loop.choose()
        new_par, new_p = ta.kv_reroot(kd, vd, P, parent, path, surv)
        torch.cuda.synchronize()
        ref = oracle.tree_attn_dense_ref(W.to_f64(q), W.bits_to_f64(kb[0]), W.bits_to_f64(vb[0]), P, parent, hkv)
        worst = max(worst, check_close(W.to_f64(out), ref, "bf16", f"iteration {it}"))
        kb, vb, want_p, want_par = oracle.kv_reroot_ref(kb, vb, P, parent, path, surv)
        assert (new_par, new_p) == (want_par, want_p), it
        keep, kr, vr = loop.advance(surv, new_par, new_p)
        kd[:, :, new_p + keep:new_p + cfg["n_tree"]] = kr.cuda()
        vd[:, :, new_p + keep:new_p + cfg["n_tree"]] = vr.cuda()
        kb[:, :, new_p + keep:new_p + cfg["n_tree"]] = W.raw_bits(kr)
        vb[:, :, new_p + keep:new_p + cfg["n_tree"]] = W.raw_bits(vr)
        if it % 20 == 0:
            print(f"[draft-loop] iteration {it} P={P} path={len(path)} survivors={len(surv)} "
                  f"max-abs={worst:.3g}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    assert loop.prefix_len > cfg["prefix"]
    assert np.array_equal(W.raw_bits(kd), kb) and np.array_equal(W.raw_bits(vd), vb)
