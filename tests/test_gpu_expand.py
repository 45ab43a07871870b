"""GPU parity of the maximum-likelihood expansion step against the CPU oracle.

The new nodes are integer decisions taken on fp32 scores (the kernel sums the
log-sum-exp in fp32), the oracle's in fp64. The test therefore compares what
is unique: when the oracle's k-th and (k+1)-th best scores are further apart
than the fp32 error bound, the (leaf, token) list must be identical; inside a
near-tie, it checks that the kernel's choice is a valid top k. Scores must
agree to the bound.

Error bound of a score: the log-sum-exp of up to 2^18 logits sums per thread,
then pairwise, in fp32 (relative error of the sum below (16 + 18) * 2^-24,
about 2e-6, so about 2e-6 absolute on its log), exp2 and log are within a
few ulp, and the final additions round at |score| * 2^-24: TOL = 5e-5 +
1e-6 * |score| leaves a wide margin.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import tree_masked_attention_attn_amd as ta
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def tol(score):
    return 5e-5 + 1e-6 * abs(score) if np.isfinite(score) else 0.0


def check(logits, scores, k, what, stride_pad=0):
    w, vocab = logits.shape
    if stride_pad:
        big = torch.full((w, vocab + stride_pad), float("nan"), dtype=logits.dtype)  # padding never read
        big[:, :vocab] = logits
        dev_logits = big.to(DEV)[:, :vocab]
    else:
        dev_logits = logits.to(DEV)
    leaf, tok, sc = ta.tree_expand(dev_logits, scores.to(DEV), k)
    torch.cuda.synchronize()
    got = list(zip(leaf.cpu().tolist(), tok.cpu().tolist()))
    got_s = sc.cpu().tolist()
    x64, s64 = W.to_f64(logits), scores.numpy().astype(np.float64)
    want = oracle.tree_expand_ref(x64, s64, k)
    ranked = sorted((c[2] for c in want), reverse=True)
    kth = ranked[-1]
    nxt = None
    if k < w * vocab:
        more = sorted((c[2] for c in oracle.tree_expand_ref(x64, s64, k + 1)), reverse=True)
        nxt = more[k]
    logp = oracle.log_softmax_rows(x64)
    leaves = [i for i, _ in got]
    assert len(set(got)) == k and leaves == sorted(leaves), f"{what}: not k distinct nodes in leaf order"
    for (i, t), s in zip(got, got_s):
        ref = s64[i] + logp[i, t]
        assert abs(s - ref) <= tol(ref) or (s == ref), f"{what}: score of ({i}, {t}) {s} vs {ref}"
    if nxt is None or kth - nxt > 2 * tol(kth):
        assert got == [(i, t) for i, t, _ in want], f"{what}: {got[:8]} != {[(i, t) for i, t, _ in want][:8]}"
        return "exact"
    # near-tie at the boundary: a valid top k (every pick at least the k-th
    # best within the bound; per leaf, a prefix of its token ranking)
    for (i, t) in got:
        assert s64[i] + logp[i, t] >= kth - 2 * tol(kth), f"{what}: ({i}, {t}) is not among the best"
    for i in set(i for i, _ in got):
        picks = [t for j, t in got if j == i]
        assert picks == [int(t) for t in oracle.token_ranking(x64[i])[:len(picks)]], f"{what}: leaf {i} not a prefix"
    return "near-tie"


@pytest.mark.parametrize("name", ["draft_expand_w8", "qwen2_72b_32k_verify", "llama3_70b_verify"])
@pytest.mark.parametrize("w,k", [(8, 8), (1, 8), (8, 1), (64, 16), (3, 16), (16, 4), (13, 5)])
def test_expand_parity(name, w, k):
    # w * k = 64 is the largest final choice made by rank (one candidate per
    # lane); 65 and above merge the leaves' lists
    cfg = W.config(name)
    rng = np.random.default_rng(cfg["seed"] * 100 + w * 17 + k)
    x = W.make_expand_inputs(cfg, w, rng)
    say(f"[expand] {name} vocab={cfg['vocab']} w={w} k={k} {cfg['dtype']}")
    check(x["logits"], x["path_scores"], k, f"{name} w={w} k={k}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("vocab", [1, 2, 7, 100, 4095, 4097, 8192, 262144])
def test_ragged_and_extreme_vocab_sizes(dtype, vocab):
    rng = np.random.default_rng(vocab)
    w = 5
    k = min(16, w * vocab)
    x = W.make_expand_inputs(dict(seed=vocab, vocab=vocab, dtype=dtype), w, rng)
    pad = (-vocab) % (8 if dtype == "bf16" else 4)
    say(f"[expand] vocab={vocab} {dtype} k={k}")
    check(x["logits"], x["path_scores"], k, f"vocab {vocab}", stride_pad=pad)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ties_infinities_and_offsets(dtype):
    """Equal logits (token-id order), equal path scores (leaf order), -inf
    logits, rows shifted by +-1000 (log-softmax does not change), one row
    with a single finite value."""
    rng = np.random.default_rng(5)
    w, vocab = 6, 10000
    x = torch.from_numpy(rng.integers(-3, 4, size=(w, vocab)).astype(np.float32))
    x[1] += 1000.0
    x[2] -= 1000.0
    x[3, ::2] = -float("inf")
    x[4].fill_(-float("inf"))
    x[4, 777] = 2.0
    x[5].fill_(1.5)  # every token equal
    s = torch.tensor([-1.0, -1.0, -2.0, -0.5, -3.0, -1.0], dtype=torch.float32)
    for k in (1, 4, 16):
        say(f"[expand] ties {dtype} k={k}")
        check(x.to(W.TORCH_DTYPE[dtype]), s, k, f"ties {dtype} k={k}")


def test_repeat_calls_reuse_the_workspace():
    rng = np.random.default_rng(6)
    ws = torch.zeros(ta.lib().ta_tree_expand_workspace_bytes(64), dtype=torch.uint8, device=DEV)
    for j, (w, vocab, k, dtype) in enumerate([(8, 128256, 8, "bf16"), (2, 52, 16, "f32"), (64, 4096, 16, "bf16"),
                                              (1, 4, 1, "f32"), (8, 128256, 8, "bf16")]):
        x = W.make_expand_inputs(dict(seed=j, vocab=vocab, dtype=dtype), w, rng)
        leaf, tok, sc = ta.tree_expand(x["logits"].to(DEV), x["path_scores"].to(DEV), k, workspace=ws)
        torch.cuda.synchronize()
        want = oracle.tree_expand_ref(W.to_f64(x["logits"]), x["path_scores"].numpy().astype(np.float64), k)
        say(f"[expand] repeat {j}: w={w} vocab={vocab} k={k}")
        assert list(zip(leaf.cpu().tolist(), tok.cpu().tolist())) == [(i, t) for i, t, _ in want], f"call {j}"
    counts = ws[:8192].view(torch.int32)
    assert int(counts.count_nonzero()) == 0  # arrival counts back at zero
