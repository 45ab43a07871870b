"""Python binding of the MI355X tree-attention library (ctypes, no compute here).

Every function marshals arguments and calls the C ABI in ``libtree_attn.so``
(declared in ``include/tree_attn.h``). torch tensors are used only as device
memory and for the current HIP stream. There is no CPU fallback: if the
library has not been built, importing works but every call raises.

    tree_attn(q, k_cache, v_cache, prefix_len, parent, layer=0, out=None)
    tree_attn_noalloc(q, k_cache, v_cache, prefix_len, parent, out)  (no workspace, no allocation)
    tree_verify(logits, tokens, parent) -> (choice, result) device tensors
    tree_expand(logits, path_scores, k) -> (leaf, token, score) device tensors
    kv_reroot(k_cache, v_cache, prefix_len, parent, accepted_path, surviving_nodes)
    tree_attn_workspace_bytes / tree_attn_num_splits / tree_attn_block_rows /
    tree_ancestor_bits / kv_reroot_plan

Layouts: q and out ``[n_tree, n_q_heads, head_dim]``; caches
``[n_layers, n_kv_heads, capacity, head_dim]``; all contiguous, same dtype
(float32 or bfloat16), on the same GPU.
"""

import ctypes
import os
import re
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtree_attn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "tree_attn.h")

TA_OK, TA_ERR_ARG, TA_ERR_UNSUPPORTED, TA_ERR_CAPACITY, TA_ERR_TREE, TA_ERR_DEVICE = range(6)
TA_F32, TA_BF16 = 0, 1
MAX_TREE = 128


class TreeAttnError(RuntimeError):
    """A call into the library returned a non-OK status."""

    def __init__(self, status, message):
        super().__init__(f"[{status}] {message}")
        self.status = status


class ta_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_layers", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()
_I32P = ctypes.POINTER(ctypes.c_int32)
_U64P = ctypes.POINTER(ctypes.c_uint64)
_CP = ctypes.POINTER(ta_kv_cache)


def lib():
    """The loaded shared library; raises if it was never built."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                   "(there is no CPU fallback)")
            L = ctypes.CDLL(LIB_PATH)
            L.ta_abi_version.restype = ctypes.c_int32
            L.ta_last_error.restype = ctypes.c_char_p
            L.ta_status_string.restype = ctypes.c_char_p
            L.ta_status_string.argtypes = [ctypes.c_int]
            L.ta_tree_attn_workspace_bytes.restype = ctypes.c_size_t
            L.ta_tree_attn_workspace_bytes.argtypes = [_CP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
            L.ta_tree_attn_num_splits.restype = ctypes.c_int32
            L.ta_tree_attn_num_splits.argtypes = [_CP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
            L.ta_tree_attn.restype = ctypes.c_int
            L.ta_tree_attn.argtypes = [ctypes.c_void_p, _CP, ctypes.c_int32, ctypes.c_int32, _I32P,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
            L.ta_tree_attn_rows.restype = ctypes.c_int
            L.ta_tree_attn_rows.argtypes = [ctypes.c_void_p, _CP, ctypes.c_int32, ctypes.c_int32, _I32P,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            L.ta_tree_attn_rows_workspace_bytes.restype = ctypes.c_size_t
            L.ta_tree_attn_rows_workspace_bytes.argtypes = [_CP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.c_int32]
            L.ta_tree_attn_rows_num_splits.restype = ctypes.c_int32
            L.ta_tree_attn_rows_num_splits.argtypes = [_CP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.c_int32]
            L.ta_tree_attn_rows_block_rows.restype = ctypes.c_int32
            L.ta_tree_attn_rows_block_rows.argtypes = [_CP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.c_int32]
            L.ta_tree_attn_rows_noalloc.restype = ctypes.c_int
            L.ta_tree_attn_rows_noalloc.argtypes = [ctypes.c_void_p, _CP, ctypes.c_int32, ctypes.c_int32, _I32P,
                                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                                    ctypes.c_void_p]
            L.ta_kv_reroot.restype = ctypes.c_int
            L.ta_kv_reroot.argtypes = [_CP, ctypes.c_int32, _I32P, ctypes.c_int32, _I32P, ctypes.c_int32,
                                       _I32P, ctypes.c_int32, _I32P, _I32P, ctypes.c_void_p]
            L.ta_tree_verify_workspace_bytes.restype = ctypes.c_size_t
            L.ta_tree_verify_workspace_bytes.argtypes = [ctypes.c_int32]
            L.ta_tree_verify.restype = ctypes.c_int
            L.ta_tree_verify.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, _I32P, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            L.ta_tree_expand_workspace_bytes.restype = ctypes.c_size_t
            L.ta_tree_expand_workspace_bytes.argtypes = [ctypes.c_int32]
            L.ta_tree_expand.restype = ctypes.c_int
            L.ta_tree_expand.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
            L.ta_set_split_wait_limit.restype = None
            L.ta_set_split_wait_limit.argtypes = [ctypes.c_int32]
            L.ta_tree_ancestor_bits.restype = ctypes.c_int
            L.ta_tree_ancestor_bits.argtypes = [_I32P, ctypes.c_int32, _U64P]
            L.ta_tree_ancestor_bitset.restype = ctypes.c_int
            L.ta_tree_ancestor_bitset.argtypes = [_I32P, ctypes.c_int32, _U64P]
            L.ta_kv_reroot_plan.restype = ctypes.c_int
            L.ta_kv_reroot_plan.argtypes = [ctypes.c_int32, ctypes.c_int32, _I32P, ctypes.c_int32, _I32P,
                                            ctypes.c_int32, _I32P, ctypes.c_int32, _I32P, _I32P, _I32P]
            if L.ta_abi_version() != 1:
                raise RuntimeError("libtree_attn.so ABI version mismatch")
            _lib = L
    return _lib


def header_symbols():
    """Names of the functions ``include/tree_attn.h`` declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(ta_[a-z_]+)\s*\(", text)))


def _check(status):
    if status != TA_OK:
        L = lib()
        raise TreeAttnError(status, f"{L.ta_status_string(status).decode()}: {L.ta_last_error().decode()}")


def _i32(seq):
    seq = [int(x) for x in seq]
    arr = (ctypes.c_int32 * max(len(seq), 1))(*seq)
    return arr, len(seq)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return TA_F32
    if t.dtype == torch.bfloat16:
        return TA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _cache_desc(k_cache, v_cache, need_device=True):
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [n_layers, n_kv_heads, capacity, head_dim] tensor")
        if need_device and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must match in shape and dtype")
    L, H, C, D = k_cache.shape
    return ta_kv_cache(k_cache.data_ptr(), v_cache.data_ptr(), L, H, C, D, _dtype_code(k_cache))


def _stream_ptr(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_workspaces = {}
_ws_lock = threading.Lock()


def _workspace(device, nbytes, kind="attn", stream=None):
    """A zero-filled workspace per (kind, device, stream), grown on demand and
    kept for reuse.

    Every call leaves the counters ready for the next (arrival counts back at
    zero), so reuse needs no clearing. Calls on one stream are ordered, so they
    may share one workspace; two streams of a device must not (their launches
    may overlap and would share arrival counts and partial rows), hence the
    stream in the key. ``stream`` is the HIP stream handle (an int); None
    means torch's current stream of ``device``. Attention, verification and
    expansion keep separate ones.
    """
    if nbytes == 0:
        return None
    dev = torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    key = (kind, dev.type, dev.index, int(stream))
    with _ws_lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.zeros(max(nbytes, 1 << 20 if kind == "attn" else 16384), dtype=torch.uint8, device=dev)
            _workspaces[key] = ws
    return ws


def tree_attn_workspace_bytes(k_cache, v_cache, n_q_heads, prefix_len, n_tree, q_first=0):
    desc = _cache_desc(k_cache, v_cache, need_device=False)
    return lib().ta_tree_attn_rows_workspace_bytes(ctypes.byref(desc), n_q_heads, prefix_len, n_tree, q_first)


def tree_attn_num_splits(k_cache, v_cache, n_q_heads, prefix_len, n_tree, q_first=0):
    desc = _cache_desc(k_cache, v_cache, need_device=False)
    return lib().ta_tree_attn_rows_num_splits(ctypes.byref(desc), n_q_heads, prefix_len, n_tree, q_first)


def tree_attn_block_rows(k_cache, v_cache, n_q_heads, prefix_len, n_tree, q_first=0):
    desc = _cache_desc(k_cache, v_cache, need_device=False)
    return lib().ta_tree_attn_rows_block_rows(ctypes.byref(desc), n_q_heads, prefix_len, n_tree, q_first)


def tree_attn(q, k_cache, v_cache, prefix_len, parent, layer=0, out=None, workspace=None, q_first=0):
    """Tree-masked attention of one layer; returns ``out`` (allocated if None).

    ``parent`` is a host sequence of ints. With ``q_first > 0`` the queries
    (and the output rows) are only the tree nodes ``q_first ..`` (the
    draft-expansion step): ``q`` is ``[len(parent) - q_first, n_q_heads,
    head_dim]``. The launch goes on torch's current stream of q's device;
    nothing is synchronised.
    """
    if q.dim() != 3 or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous [n_rows, n_q_heads, head_dim] GPU tensor")
    desc = _cache_desc(k_cache, v_cache)
    if q.dtype != k_cache.dtype or q.device != k_cache.device:
        raise ValueError("q must match the cache in dtype and device")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    par, n = _i32(parent)
    if q.shape[0] != n - q_first:
        raise ValueError("q must have one row per tree node from q_first on")
    nbytes = lib().ta_tree_attn_rows_workspace_bytes(ctypes.byref(desc), q.shape[1], prefix_len, n, q_first)
    if workspace is None:
        workspace = _workspace(q.device, nbytes)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if q_first == 0:
        _check(lib().ta_tree_attn(q.data_ptr(), ctypes.byref(desc), layer, prefix_len, par, n, q.shape[1],
                                  out.data_ptr(), ws_ptr, ws_len, _stream_ptr(q.device)))
    else:
        _check(lib().ta_tree_attn_rows(q.data_ptr(), ctypes.byref(desc), layer, prefix_len, par, n, q_first,
                                       q.shape[1], out.data_ptr(), ws_ptr, ws_len, _stream_ptr(q.device)))
    return out


def tree_attn_noalloc(q, k_cache, v_cache, prefix_len, parent, out, layer=0, q_first=0):
    """``tree_attn`` through ``ta_tree_attn_rows_noalloc``: no workspace and no
    allocation anywhere (``out`` must be given). The split workspace is the
    library's static scratch of the current device, shared by every such
    call there; calls that can overlap on one GPU must not be issued."""
    if q.dim() != 3 or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous [n_rows, n_q_heads, head_dim] GPU tensor")
    desc = _cache_desc(k_cache, v_cache)
    if q.dtype != k_cache.dtype or q.device != k_cache.device:
        raise ValueError("q must match the cache in dtype and device")
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    par, n = _i32(parent)
    if q.shape[0] != n - q_first:
        raise ValueError("q must have one row per tree node from q_first on")
    _check(lib().ta_tree_attn_rows_noalloc(q.data_ptr(), ctypes.byref(desc), layer, prefix_len, par, n, q_first,
                                           q.shape[1], out.data_ptr(), _stream_ptr(q.device)))
    return out


def tree_verify(logits, tokens, parent, choice=None, result=None, workspace=None):
    """Greedy verification of a draft tree; returns ``(choice, result)``.

    ``logits`` is a GPU tensor ``[n_tree + 1, vocab]`` (float32 or bfloat16;
    rows may be strided, elements contiguous): row 0 is the target at the
    last verified token, row ``1 + i`` at tree node ``i``. ``tokens`` is an
    int32 GPU tensor ``[n_tree]`` of drafted tokens; ``parent`` a host
    sequence. ``choice`` ``[n_tree + 1]`` receives each row's arg-max and
    ``result`` ``[n_tree + 2]`` receives ``[m, bonus, path..., -1...]``
    (both int32 on the GPU, allocated if None). Enqueued on torch's current
    stream; nothing is synchronised (``accepted`` reads the result back).
    """
    if logits.dim() != 2 or not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a [n_tree + 1, vocab] GPU tensor with contiguous rows")
    par, n = _i32(parent)
    if logits.shape[0] != n + 1:
        raise ValueError("logits must have one row for the root and one per tree node")
    if tokens.dtype != torch.int32 or tokens.shape != (n,) or not tokens.is_contiguous() or \
            tokens.device != logits.device:
        raise ValueError("tokens must be a contiguous int32 tensor [n_tree] on the logits' device")
    dev = logits.device
    if choice is None:
        choice = torch.empty(n + 1, dtype=torch.int32, device=dev)
    if result is None:
        result = torch.empty(n + 2, dtype=torch.int32, device=dev)
    for name, t, size in (("choice", choice, n + 1), ("result", result, n + 2)):
        if t.dtype != torch.int32 or t.shape != (size,) or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous int32 tensor [{size}] on the logits' device")
    nbytes = lib().ta_tree_verify_workspace_bytes(n)
    if nbytes == 0:
        _check(TA_ERR_UNSUPPORTED)
    if workspace is None:
        workspace = _workspace(dev, nbytes, kind="verify")
    ws_len = workspace.numel() * workspace.element_size()
    _check(lib().ta_tree_verify(logits.data_ptr(), _dtype_code(logits), logits.shape[1], logits.stride(0),
                                tokens.data_ptr() if n else None, par, n, choice.data_ptr(), result.data_ptr(),
                                workspace.data_ptr(), ws_len, _stream_ptr(dev)))
    return choice, result


def tree_expand(logits, path_scores, k, leaf=None, token=None, score=None, workspace=None):
    """One maximum-likelihood expansion step; returns ``(leaf, token, score)``.

    ``logits`` is a GPU tensor ``[w, vocab]`` (float32 or bfloat16; rows may be
    strided, elements contiguous) of the draft model's logits after each
    frontier leaf; ``path_scores`` a float32 GPU tensor ``[w]``. The outputs
    (int32, int32, float32 GPU tensors ``[k]``, allocated if None) list the
    ``k`` best children by (leaf, slot). Enqueued on torch's current stream;
    nothing is synchronised.
    """
    if logits.dim() != 2 or not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a [w, vocab] GPU tensor with contiguous rows")
    w = logits.shape[0]
    dev = logits.device
    if path_scores.dtype != torch.float32 or path_scores.shape != (w,) or not path_scores.is_contiguous() or \
            path_scores.device != dev:
        raise ValueError("path_scores must be a contiguous float32 tensor [w] on the logits' device")
    k = int(k)
    leaf = torch.empty(k, dtype=torch.int32, device=dev) if leaf is None else leaf
    token = torch.empty(k, dtype=torch.int32, device=dev) if token is None else token
    score = torch.empty(k, dtype=torch.float32, device=dev) if score is None else score
    for name, t, dt in (("leaf", leaf, torch.int32), ("token", token, torch.int32), ("score", score, torch.float32)):
        if t.dtype != dt or t.shape != (k,) or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous {dt} tensor [k] on the logits' device")
    nbytes = lib().ta_tree_expand_workspace_bytes(w)
    if nbytes == 0:
        _check(TA_ERR_UNSUPPORTED)
    if workspace is None:
        workspace = _workspace(dev, nbytes, kind="expand")
    ws_len = workspace.numel() * workspace.element_size()
    _check(lib().ta_tree_expand(logits.data_ptr(), _dtype_code(logits), logits.shape[1], logits.stride(0),
                                path_scores.data_ptr(), w, k, leaf.data_ptr(), token.data_ptr(), score.data_ptr(),
                                workspace.data_ptr(), ws_len, _stream_ptr(dev)))
    return leaf, token, score


def accepted(result):
    """``(path, bonus)`` from a ``tree_verify`` result (copies it to the host)."""
    r = result.cpu().tolist()
    return r[2:2 + r[0]], r[1]


def kv_reroot(k_cache, v_cache, prefix_len, parent, accepted_path, surviving_nodes):
    """Re-root every layer in place; returns ``(new_parent, new_prefix_len)``.

    The row moves are enqueued on torch's current stream of the cache's device.
    """
    desc = _cache_desc(k_cache, v_cache)
    par, n = _i32(parent)
    path, m = _i32(accepted_path)
    surv, ns = _i32(surviving_nodes)
    new_par = (ctypes.c_int32 * max(ns, 1))()
    new_p = ctypes.c_int32(0)
    _check(lib().ta_kv_reroot(ctypes.byref(desc), prefix_len, par, n, path, m, surv, ns, new_par,
                              ctypes.byref(new_p), _stream_ptr(k_cache.device)))
    return [new_par[i] for i in range(ns)], new_p.value


def set_split_wait_limit(polls):
    """Bound (in polls about 2048 GPU cycles apart) of the wait between prefix splits."""
    lib().ta_set_split_wait_limit(int(polls))


def tree_ancestor_bits(parent):
    """Host-only: bit j of entry i is set iff node j is i or an ancestor of i
    (Python ints of up to 128 bits, from the two-word C bitsets)."""
    par, n = _i32(parent)
    words = (ctypes.c_uint64 * max(2 * n, 1))()
    _check(lib().ta_tree_ancestor_bitset(par, n, words))
    return [words[2 * i] | (words[2 * i + 1] << 64) for i in range(n)]


def kv_reroot_plan(prefix_len, capacity, parent, accepted_path, surviving_nodes):
    """Host-only re-root plan: ``(src_rows, new_parent, new_prefix_len)``."""
    par, n = _i32(parent)
    path, m = _i32(accepted_path)
    surv, ns = _i32(surviving_nodes)
    src = (ctypes.c_int32 * max(m + ns, 1))()
    new_par = (ctypes.c_int32 * max(ns, 1))()
    new_p = ctypes.c_int32(0)
    _check(lib().ta_kv_reroot_plan(prefix_len, capacity, par, n, path, m, surv, ns, src, new_par,
                                   ctypes.byref(new_p)))
    return [src[i] for i in range(m + ns)], [new_par[i] for i in range(ns)], new_p.value
