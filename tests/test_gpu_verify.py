"""GPU parity of greedy tree verification against the CPU oracle (bit-exact).

The HIP path (through the C ABI) must reproduce the oracle's per-row arg-max
and its ``[m, bonus, path..., -1...]`` result exactly: this is integer work,
and the arg-max decisions are taken on the stored values on both sides.
"""

import sys
import zlib

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


def expected(logits, tokens, parent):
    path, bonus, choice = oracle.tree_verify_ref(W.to_f64(logits), np.asarray(tokens), parent)
    n = len(parent)
    return list(map(int, choice)), [len(path), bonus] + list(path) + [-1] * (n - len(path))


def check(logits, tokens, parent, what, stride_pad=0):
    n = len(parent)
    if stride_pad:
        big = torch.empty((n + 1, logits.shape[1] + stride_pad), dtype=logits.dtype)
        big.fill_(float("nan"))  # the padding is never read
        big[:, :logits.shape[1]] = logits
        dev_logits = big.to(DEV)[:, :logits.shape[1]]
    else:
        dev_logits = logits.to(DEV)
    tok = torch.as_tensor(np.asarray(tokens, dtype=np.int32)).to(DEV)
    choice, result = ta.tree_verify(dev_logits, tok, parent)
    torch.cuda.synchronize()
    want_choice, want_result = expected(logits, tokens, parent)
    assert choice.cpu().tolist() == want_choice, f"{what}: arg-max differs"
    assert result.cpu().tolist() == want_result, f"{what}: result {result.cpu().tolist()[:12]} != {want_result[:12]}"
    return want_result[0]


@pytest.mark.parametrize("name", ["llama3_70b_verify", "llama3_70b_verify_bs8", "qwen2_72b_32k_verify",
                                  "llama3_8b_verify", "tiny_fp32"])
@pytest.mark.parametrize("accept", [0.0, 0.8, 1.0])
def test_config_verify_parity(name, accept):
    cfg = W.config(name)
    parent, _ = W.make_tree(cfg, np.random.default_rng(cfg["seed"]))
    say(f"[verify] {name} n={len(parent)} vocab={cfg['vocab']} {cfg['dtype']} accept={accept}")
    x = W.make_verify_inputs(cfg, parent, np.random.default_rng(cfg["seed"] + int(accept * 10)), accept=accept)
    m = check(x["logits"], x["tokens"], parent, f"{name} accept={accept}")
    if accept == 0.0:
        assert m == 0
    if accept == 1.0:
        assert m >= 1


def _rand_parent(rng, n):
    return [-1] + [int(rng.integers(-1, i)) for i in range(1, n)] if n else []


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("vocab", [1, 3, 7, 9, 33, 1000, 4099, 16385, 128256])
def test_ragged_vocab_sizes(dtype, vocab):
    rng = np.random.default_rng(vocab)
    parent = _rand_parent(rng, 13)
    cfg = dict(seed=vocab, vocab=vocab, dtype=dtype)
    say(f"[verify] vocab={vocab} {dtype}")
    x = W.make_verify_inputs(cfg, parent, rng, accept=0.9)
    pad = (-vocab) % (8 if dtype == "bf16" else 4)
    if pad == 0:
        check(x["logits"], x["tokens"], parent, f"vocab {vocab}")
    else:
        check(x["logits"], x["tokens"], parent, f"vocab {vocab} strided", stride_pad=pad)


def _deep_parent(rng, n):
    return [-1] + [max(-1, i - 1 - int(rng.integers(0, 3))) for i in range(1, n)]


@pytest.mark.parametrize("shape", ["root_only", "chain64", "forest64", "random64", "strided", "chain128",
                                   "forest128", "random128", "deep128", "deep100"])
def test_tree_shapes(shape):
    rng = np.random.default_rng(zlib.crc32(shape.encode()))
    parent = {"root_only": [], "chain64": [-1] + list(range(63)), "forest64": [-1] * 64,
              "random64": _rand_parent(rng, 64), "strided": _rand_parent(rng, 40),
              "chain128": [-1] + list(range(127)), "forest128": [-1] * 128, "random128": _rand_parent(rng, 128),
              "deep128": _deep_parent(rng, 128), "deep100": _deep_parent(rng, 100)}[shape]
    cfg = dict(seed=1, vocab=5000, dtype="bf16")
    say(f"[verify] shape {shape} n={len(parent)}")
    for accept in (0.5, 0.97, 1.0):
        x = W.make_verify_inputs(cfg, parent, rng, accept=accept)
        check(x["logits"], x["tokens"], parent, f"{shape} accept={accept}", stride_pad=24 if shape == "strided" else 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ties_signed_zeros_and_infinities(dtype):
    """Equal maxima across workgroups, -0.0 against +0.0, all -inf rows,
    the maximum in the ragged tail: every arg-max is the first maximum."""
    vocab = 40000 + 5
    n = 7
    parent = [-1, 0, 0, 1, -1, 4, 5]
    tdt = W.TORCH_DTYPE[dtype]
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((n + 1, vocab), dtype=np.float32)).to(tdt)
    x[0, 30000] = 100.0; x[0, 39000] = 100.0; x[0, 35000] = 100.0   # same maximum, far apart
    x[1].fill_(-float("inf"))                                         # every value -inf
    x[2].fill_(-1.0); x[2, 100] = -0.0; x[2, 20000] = 0.0            # -0.0 == +0.0: index 100 first
    x[3].fill_(-float("inf")); x[3, vocab - 1] = float("inf")         # +inf in the tail
    x[4].zero_()                                                      # all equal
    x[5, vocab - 2] = 50.0; x[5, vocab - 1] = 50.0                    # tie inside the tail
    x[6].fill_(3.0); x[6, 0] = -1.0                                   # tie everywhere but index 0
    x[7, 17] = float("inf"); x[7, 16] = float("inf")
    choice = [int(v) for v in oracle.row_argmax(W.to_f64(x))]
    assert choice[:3] == [30000, 0, 100]
    tokens = [choice[0 if p < 0 else p + 1] for p in parent]  # the whole tree agrees
    say(f"[verify] ties {dtype}")
    m = check(x, tokens, parent, f"ties {dtype}", stride_pad=3)  # rows of 40008 values
    assert m == 3


def test_repeat_calls_reuse_the_workspace():
    """Calls of different shapes in a row on one workspace; each must match."""
    rng = np.random.default_rng(3)
    ws = torch.zeros(16384, dtype=torch.uint8, device=DEV)
    for k, (n, vocab, dtype) in enumerate([(64, 128256, "bf16"), (3, 100, "f32"), (0, 80, "bf16"),
                                           (64, 152064, "bf16"), (17, 9000, "f32"), (64, 128256, "bf16")]):
        parent = _rand_parent(rng, n)
        x = W.make_verify_inputs(dict(seed=k, vocab=vocab, dtype=dtype), parent, rng, accept=0.9)
        tok = x["tokens"].to(DEV)
        say(f"[verify] repeat {k}: n={n} vocab={vocab} {dtype}")
        choice, result = ta.tree_verify(x["logits"].to(DEV), tok, parent, workspace=ws)
        torch.cuda.synchronize()
        want_choice, want_result = expected(x["logits"], x["tokens"], parent)
        assert choice.cpu().tolist() == want_choice and result.cpu().tolist() == want_result, f"call {k}"
    assert int(ws.count_nonzero()) == 0  # left zero for the next call


def test_verify_feeds_reroot():
    """The device result drives the re-root: accepted path into the prefix,
    the subtree below the last accepted node survives."""
    cfg = W.config("llama3_8b_verify", prefix=300)
    x = W.make_inputs(cfg)
    parent, P = x["parent"], x["prefix_len"]
    v = W.make_verify_inputs(cfg, parent, np.random.default_rng(4), accept=0.9)
    _, result = ta.tree_verify(v["logits"].to(DEV), v["tokens"].to(DEV), parent)
    path, bonus = ta.accepted(result)
    want_path, want_bonus, _ = oracle.tree_verify_ref(W.to_f64(v["logits"]), v["tokens"].numpy(), parent)
    assert (path, bonus) == (want_path, want_bonus)
    surv = W.descendants(parent, path[-1]) if path else list(range(len(parent)))
    say(f"[verify] -> reroot path={path} survivors={len(surv)}")
    k, vv = x["k"].to(DEV), x["v"].to(DEV)
    kb, vb = W.raw_bits(x["k"]), W.raw_bits(x["v"])
    new_par, new_p = ta.kv_reroot(k, vv, P, parent, path, surv)
    torch.cuda.synchronize()
    k2, v2, want_p, want_par = oracle.kv_reroot_ref(kb, vb, P, parent, path, surv)
    assert (new_par, new_p) == (want_par, want_p)
    assert np.array_equal(W.raw_bits(k), k2) and np.array_equal(W.raw_bits(vv), v2)
