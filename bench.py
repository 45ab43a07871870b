"""Benchmark of the tree-attention hot path on one MI355X.

One step = one ``tree_attn`` call (one layer of a verify step) followed by one
``kv_reroot`` of the same cache (an accepted path of 1..8 nodes and its
surviving subtree), i.e. the whole path once. The default workload is the
Llama-3-70B-shaped verify: 64 query / 8 KV heads, head_dim 128, bf16, prefix
8192, a 64-node width-8 tree; synthetic seeded inputs.

Labelled extras, outside the step (``--no-extras`` skips them): ``tree_verify``
(greedy verification of the same tree against the target's logits over the
model's vocabulary), ``tree_expand`` (one maximum-likelihood expansion step:
8 frontier leaves, 8 new nodes, over the same vocabulary) and
``kv_reroot_all_layers`` (one re-root call over a cache with all of the
model's layers, for the path the verification accepted: the draft side with
its survivors, and the target side with the accepted rows only).

Timing: inputs are resident in HBM before the timed region. ``--rotate`` input
sets are cycled so that the working set exceeds twice the 256 MB Infinity
Cache (each set is one layer's K/V, as in a real step where the other layers
have evicted it). A short device sleep is queued first so the host runs ahead
and the kernels execute back to back. HIP events on the launch stream
(created without the system-scope fence, so that recording them writes back
no caches) bracket the timed region of K whole steps (-> ms_per_step), then K
launches of each
kernel alone, each between its own events (-> its mean launch duration, which
the roofline uses, and the spread), then the same launches back to back
(-> the launch period, dispatch gaps included). Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

Counter support (the traffic figure of the roofline):
    --copy-calib        also run one plain 256 MiB device copy (the
                        FETCH_SIZE / WRITE_SIZE calibration kernel)
    --summarize DIR OUT turn rocprofv3 output under DIR (kernel-trace stats or
                        counter CSVs) into the text summary OUT and exit
"""

import argparse
import ctypes
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

# The headline metric, as the benchmark definition names it.
METRIC = "tree-attn \u00b5s/step + achieved HBM GB/s (frac of peak); kv_reroot GB/s"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 vector
MALL_BYTES = 256 << 20
COPY_BYTES = 256 << 20     # calibration copy size
KERNEL_SOURCES = ["tree_masked_attention_attn_amd/csrc/tree_attn_kernel.hip",
                  "tree_masked_attention_attn_amd/csrc/plan.cpp",
                  "tree_masked_attention_attn_amd/csrc/plan.h",
                  "tree_masked_attention_attn_amd/csrc/api.cpp"]
PROFILES = os.path.join(ROOT, "profiles")


# --------------------------------------------------------------------------
# Timing events: HIP events created with hipEventDisableSystemFence, recorded
# on the launch stream. The default events of torch add a system-scope cache
# write-back and invalidation at every record, which lengthens the measured
# interval of short kernels by 1-3 us and slows the work after it; these
# record a timestamp only (the HIP runtime documents the flag for timing).

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_HIP = None


def _hip():
    """The HIP runtime the process already uses (torch's), for its events."""
    global _HIP
    if _HIP is None:
        import torch
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        L = ctypes.CDLL(path)
        L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = L
    return _HIP


class Ev:
    """A timing event on a torch stream (record, then elapsed_time in ms)."""

    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = _hip().hipEventCreateWithFlags(ctypes.byref(self.h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = _hip().hipEventRecord(self.h, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = _hip().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self.h and _HIP is not None:
            _HIP.hipEventDestroy(self.h)


def kernel_source_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def tree_attn_work(cfg, parent):
    """Algorithmic bytes and flops of one tree_attn call.

    bytes: K and V rows of the prefix and the tree (read once per KV head),
    q in, out back, the parent array. flops: 2 (QK) + 2 (PV) per visible
    (row, key) pair and head_dim element; the tree block counts only visible
    pairs (ancestors and self).
    """
    P, n, hq, hkv, d = cfg["prefix"], cfg["n_tree"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    qf = cfg.get("q_first", 0)  # query rows: nodes qf .. n-1
    es = 4 if cfg["dtype"] == "f32" else 2
    anc = 0
    for i in range(qf, n):
        j = i
        while j != -1:
            anc += 1
            j = parent[j]
    nbytes = 2 * hkv * d * es * (P + n) + 2 * (n - qf) * hq * d * es + 4 * n
    flops = 4 * d * hq * ((n - qf) * P + anc)
    return nbytes, flops, anc


def reroot_bytes(cfg, src_rows, prefix, n_layers=1):
    """Algorithmic bytes of one kv_reroot: read + write of every moved row."""
    es = 4 if cfg["dtype"] == "f32" else 2
    moved = sum(1 for k, s in enumerate(src_rows) if s != prefix + k)
    return 2 * moved * 2 * cfg["n_kv_heads"] * cfg["head_dim"] * es * n_layers


def split_partial_bytes(cfg, splits, block_rows):
    """Bytes of split partials one tree_attn launch writes (and the merge
    reads back once): per unit and written row, a (max, sum) fp32 pair and O
    in fp32. A unit writes its block's rows (block_rows of them, 128 or 64);
    the bf16 kernel skips the 32-row tiles that lie wholly past the head's
    last query row. Overhead, not algorithmic."""
    if splits <= 1:
        return 0
    rows = cfg["n_q_heads"] // cfg["n_kv_heads"] * (cfg["n_tree"] - cfg.get("q_first", 0))
    written = 0
    for rb in range(-(-rows // block_rows)):
        block = min(block_rows, rows - block_rows * rb)
        written += block_rows if cfg["dtype"] == "f32" else 32 * -(-block // 32)
    return cfg["n_kv_heads"] * splits * written * (8 + cfg["head_dim"] * 4)


def verify_bytes(cfg, n):
    """Algorithmic bytes of one tree_verify: every logits value once, the
    drafted tokens, the arg-max and result arrays."""
    es = 4 if cfg["dtype"] == "f32" else 2
    return (n + 1) * cfg["vocab"] * es + 4 * n + 4 * (n + 1) + 4 * (n + 2)


def expand_bytes(cfg, w, k):
    """Algorithmic bytes of one tree_expand: every logit once, the path
    scores and the three k-entry outputs."""
    es = 4 if cfg["dtype"] == "f32" else 2
    return w * cfg["vocab"] * es + 4 * w + 12 * k


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))]


def traffic_file(cfg):
    return os.path.join(PROFILES, f"tree_attn_{cfg['dtype']}_{cfg['name']}_traffic.txt")


def load_traffic(cfg):
    """HBM bytes per tree_attn launch from the committed counter summary, or
    None when there is none or the kernel sources changed since."""
    path = traffic_file(cfg)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.loads(f.read().split("```json", 1)[1].split("```", 1)[0])
    if rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("traffic_bytes")


def cpu_baseline(cfg, x, path, surv, budget_s, budget_1t=0.0):
    """The oracle as it stands, on a bounded sample of the same workload: with
    BLAS threads on every host core (the reported value), and again with one
    thread (value_1thread) on a smaller sample."""
    from threadpoolctl import threadpool_limits

    import oracle
    cores = len(os.sched_getaffinity(0))
    q = W.to_f64(x["q"])
    k = W.to_f64(x["k"][0])
    v = W.to_f64(x["v"][0])
    P, parent, n = x["prefix_len"], x["parent"], cfg["n_tree"]
    qf = x.get("q_first", 0)
    rows = n - qf
    kb, vb = W.raw_bits(x["k"]), W.raw_bits(x["v"])

    def sample(threads, budget):
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            done = 0
            # one query node at a time (its own ancestors only), until the time budget is spent
            while done < rows and time.perf_counter() - t0 < budget:
                _one_node(oracle, q, k, v, P, parent, qf, qf + done, cfg["n_kv_heads"])
                done += 1
            attn_s = (time.perf_counter() - t0) / done
            t1 = time.perf_counter()
            oracle.kv_reroot_ref(kb, vb, P, parent, path, surv)
            reroot_s = time.perf_counter() - t1
        return (attn_s * rows + reroot_s) * 1e6, done

    step_us, done = sample(cores, budget_s)
    res = {"value": round(step_us, 1), "unit": "us/step", "cores": cores, "kind": "oracle",
           "sample": f"tree_attn_ref on {done} of {rows} query nodes (all heads, full prefix), scaled "
                     f"x{rows / done:.2f} to all of them, plus one kv_reroot_ref of the same cache; numpy fp64"}
    if budget_1t > 0:
        one_us, done1 = sample(1, budget_1t)
        res["value_1thread"] = round(one_us, 1)
        res["sample_1thread"] = f"the same with one BLAS thread on {done1} of {rows} query nodes"
    return res


def _one_node(oracle, q, k, v, P, parent, qf, i, hkv):
    """Output of query node i alone: the oracle on the tree truncated after
    node i (its ancestors all precede it), with node i as the only query."""
    r = i - qf
    return oracle.tree_attn_ref(q[r: r + 1], k, v, P, parent[: i + 1], hkv, q_first=i)[0]


# --------------------------------------------------------------------------
# rocprofv3 output -> committed text summaries


def _rows(d, pattern):
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True)):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def summarize(d, out_path, command):
    lines = [f"# rocprofv3 summary: {os.path.basename(out_path)}", "",
             f"Attention kernel sources (sha256, first 16 hex digits of {', '.join(os.path.basename(k) for k in KERNEL_SOURCES)}): "
             f"{kernel_source_sha()}", "", "Command (from the repository root):", "", "```", command, "```", ""]
    stats = _rows(d, "*kernel_stats.csv")
    if stats:
        lines += ["Kernel statistics (durations in microseconds):", "",
                  "| kernel | calls | total us | average us | min us | max us | share |",
                  "|---|---|---|---|---|---|---|"]
        for r in stats:
            lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    dbs = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    if not stats and dbs:  # rocpd output: per-dispatch durations in the `kernels` view
        import sqlite3
        lines += ["Kernel statistics from the kernel trace (durations in microseconds):", "",
                  "| kernel | calls | total us | average us | min us | max us |", "|---|---|---|---|---|---|"]
        for db in dbs:
            con = sqlite3.connect(db)
            rows = list(con.execute(
                "select name, count(*), sum(duration), avg(duration), min(duration), max(duration) "
                "from kernels group by name order by sum(duration) desc"))
            for name, n, tot, avg, mn, mx in rows:
                lines.append(f"| {name[:90]} | {n} | {tot / 1e3:.1f} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
                             f"{mx / 1e3:.2f} |")
            # the library's kernels split by launch size (a re-root of all
            # layers and one of a single layer are the same kernel)
            if "grid_x" in {r[1] for r in con.execute("pragma table_info(kernels)")}:
                lines += ["", "The library's kernels by launch size (grid in threads, x by y):", "",
                          "| kernel | grid | calls | average us | min us | max us |", "|---|---|---|---|---|---|"]
                for name, gx, gy, n, avg, mn, mx in con.execute(
                        "select name, grid_x, grid_y, count(*), avg(duration), min(duration), max(duration) "
                        "from kernels group by name, grid_x, grid_y order by name, grid_x * grid_y"):
                    if any(k in name for k in ("tree_attn", "kv_reroot", "tree_verify", "tree_expand")):
                        lines.append(f"| {name[:60]} | {gx} x {gy} | {n} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
                                     f"{mx / 1e3:.2f} |")
            # where the longest dispatches of the library's kernels fall in the run
            lines += ["", "Longest dispatches of the library's kernels (n-th dispatch of that kernel, "
                      "microseconds after the run's first dispatch of any kernel):", "",
                      "| kernel | dispatch | of | duration us | at us |", "|---|---|---|---|---|"]
            cols = {r[1] for r in con.execute("pragma table_info(kernels)")}
            order = "start" if "start" in cols else "rowid"
            t_first = next(con.execute(f"select min({order}) from kernels"))[0]
            for name, n, *_ in rows:
                if not any(k in name for k in ("tree_attn", "kv_reroot", "tree_verify", "tree_expand")):
                    continue
                disp = list(con.execute(f"select duration, {order} from kernels where name = ? order by {order}",
                                        (name,)))
                top = sorted(range(len(disp)), key=lambda i: -disp[i][0])[:3]
                for i in top:
                    lines.append(f"| {name[:60]} | {i + 1} | {n} | {disp[i][0] / 1e3:.2f} | "
                                 f"{(disp[i][1] - t_first) / 1e3:.1f} |")
            con.close()
        lines.append("")
    counters = _rows(d, "*counter_collection.csv")
    if counters:
        per = {}
        for r in counters:
            name = r["Kernel_Name"]
            key = ("tree_attn" if "tree_attn" in name else "kv_reroot" if "kv_reroot" in name
                   else "copy" if "copy" in name.lower() else None)
            if key is None:
                continue
            per.setdefault((key, r["Counter_Name"]), {}).setdefault(r["Dispatch_Id"], 0.0)
            per[(key, r["Counter_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
        lines += ["Counters per dispatch (tree_attn, kv_reroot: mean over dispatches; copy: the",
                  "largest copy dispatch, which is the calibration copy):", "",
                  "| kernel | counter | dispatches | value |", "|---|---|---|---|"]
        agg = {}
        for (k, c), vals in sorted(per.items()):
            v = list(vals.values())
            # the calibration copy is the largest copy dispatch (uploads are smaller)
            agg[(k, c)] = max(v) if k == "copy" else statistics.fmean(v)
            what = "largest" if k == "copy" else "mean"
            lines.append(f"| {k} | {c} | {len(v)} | {agg[(k, c)]:.1f} ({what}) |")
        lines.append("")
        return lines, agg
    return lines, {}


def main_summarize(args):
    d, out = args.summarize
    lines, agg = summarize(d, out, args.command or "")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def main_traffic(args):
    """Combine a FETCH_SIZE and a WRITE_SIZE counter run into the traffic record."""
    fetch_dir, write_dir = args.traffic
    cfg = W.config(args.config)
    _, fa = summarize(fetch_dir, "", "")
    _, wa = summarize(write_dir, "", "")
    copy_kib = COPY_BYTES / 1024
    f_fac = fa[("copy", "FETCH_SIZE")] / copy_kib
    w_fac = wa[("copy", "WRITE_SIZE")] / copy_kib
    f_kib = fa[("tree_attn", "FETCH_SIZE")]
    w_kib = wa[("tree_attn", "WRITE_SIZE")]
    rec = {"kernel": "tree_attn", "workload": cfg["name"], "source_sha": kernel_source_sha(),
           "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
           "copy_bytes": COPY_BYTES, "copy_fetch_factor": round(f_fac, 4), "copy_write_factor": round(w_fac, 4),
           "traffic_bytes": int(round((f_kib / f_fac + w_kib / w_fac) * 1024))}
    text = ["# HBM traffic of tree_attn, " + cfg["name"], "",
            "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs, each divided by",
            f"what the same counter reads for one plain {COPY_BYTES >> 20} MiB device copy in the same process.",
            "bench.py reports traffic_bytes only while source_sha matches the kernel sources.", "",
            "Commands (from the repository root):", "", "```", args.command or "", "```", "",
            "```json", json.dumps(rec, indent=1), "```", ""]
    with open(traffic_file(cfg), "w") as f:
        f.write("\n".join(text))
    print(json.dumps(rec))


def counter_summary(dirs, command, workload=""):
    """Counter passes (rocprofv3 --pmc, CSV) over tree_attn: per-dispatch means
    and rocprofv3's own derived utilisations. The CSV sums a counter's
    instances, so GRBM_GUI_ACTIVE (one instance per XCD, where the derived
    expressions take the maximum) is divided by the XCD count."""
    means, info = {}, {}
    for d in dirs:
        _, agg = summarize(d, "", "")
        for (k, c), v in agg.items():
            if k == "tree_attn":
                means.setdefault(c, []).append(v)
        for r in _rows(d, "*agent_info.csv"):
            if r.get("Name", "").startswith("gfx"):
                info = r
    m = {c: statistics.fmean(v) for c, v in means.items()}
    xcc, cus, simds = int(info["Num_Xcc"]), int(info["Cu_Count"]), int(info["Simd_Count"])
    gui = m["GRBM_GUI_ACTIVE"] / xcc
    derived = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        derived.append(("MfmaUtil (% of SIMD cycles, GPU-active basis)",
                        100 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds)))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "SQ_INSTS_MFMA" in m:
        derived.append(("MFMA busy cycles per MFMA instruction", m["SQ_VALU_MFMA_BUSY_CYCLES"] / m["SQ_INSTS_MFMA"]))
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        derived.append(("MFMA-busy cycles in which a VALU instruction also issued (%)",
                        100 * m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"]))
    if "SQ_LDS_IDX_ACTIVE" in m:
        derived.append(("LDS indexed-access utilisation (% of CU cycles, GPU-active basis)", 100 * m["SQ_LDS_IDX_ACTIVE"] / (gui * cus)))
    if "SQ_LDS_IDX_ACTIVE" in m and "SQ_LDS_BANK_CONFLICT" in m:
        derived.append(("LDS bank-conflict cycles per conflict-free LDS cycle",
                        m["SQ_LDS_BANK_CONFLICT"] / (m["SQ_LDS_IDX_ACTIVE"] - m["SQ_LDS_BANK_CONFLICT"])))
    if "SQ_INSTS_VALU" in m and "SQ_INSTS_MFMA" in m:
        derived.append(("VALU instructions per MFMA instruction", m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"]))
    lines = ["# rocprofv3 counters: tree_attn" + (", " + workload if workload else ""), "",
             f"Attention kernel sources (sha256, first 16 hex digits): {kernel_source_sha()}", "",
             "Commands (from the repository root):", "", "```", command, "```",
             "", f"Part: {info.get('Name', '?')}, {cus} CUs, {simds} SIMDs, {xcc} XCDs. Means per tree_attn dispatch "
             "(all instances summed):", "", "| counter | value |", "|---|---|"]
    lines += [f"| {c} | {v:.1f} |" for c, v in sorted(m.items())]
    lines += ["", "Derived (rocprofv3's expressions; GRBM_GUI_ACTIVE per XCD):", "", "| metric | value |", "|---|---|"]
    lines += [f"| {name} | {v:.3f} |" for name, v in derived]
    return lines + [""], m, dict(derived)


def main_counters(args):
    out, dirs = args.counters[0], args.counters[1:]
    lines, _, _ = counter_summary(dirs, args.command or "", args.config)
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}")


def run_extras(ta, torch, cfg, dev, parent, P, K, timed):
    """The labelled extras: verification, expansion, all-layer re-root."""
    # Verification of the same tree against the target's logits: rotated
    # logits sets (positive rescales of one draw, so the same tokens apply)
    # that together exceed twice the Infinity Cache.
    n = cfg["n_tree"]
    vx = W.make_verify_inputs(cfg, parent)
    v_bytes = verify_bytes(cfg, n)
    vrot = max(2, math.ceil(2 * MALL_BYTES / v_bytes) + 1)
    v0 = vx["logits"].to(dev)
    v_sets = [v0 * (1.0 + 1e-3 * r) if r else v0 for r in range(vrot)]
    v_tok = vx["tokens"].to(dev)
    v_choice = torch.empty(n + 1, dtype=torch.int32, device=dev)
    v_result = torch.empty(n + 2, dtype=torch.int32, device=dev)
    v_ws = torch.zeros(16384, dtype=torch.uint8, device=dev)

    def verify(i):
        ta.tree_verify(v_sets[i % vrot], v_tok, parent, choice=v_choice, result=v_result, workspace=v_ws)

    for i in range(5):
        verify(i)
    _, ver_us, _ = timed(verify, K, each=True)
    ver_b2b, _, _ = timed(verify, K)
    # logits still in the caches, as when the LM head has just written them
    _, ver_hot, _ = timed(lambda i: verify(0), 50, each=True)
    v_path = ta.accepted(v_result)[0]
    del v_sets, v0

    # One re-root call over a cache with all of the model's layers, for the
    # path the verification above accepted: the draft side keeps the subtree
    # below its last node, the target side only the accepted rows. The
    # prefix position rotates (P, P - n, ...) so that the rows touched by
    # consecutive calls differ and together exceed twice the Infinity Cache.
    n_layers = cfg.get("layers", 1)
    big = (n_layers, cfg["n_kv_heads"], cfg["capacity"], cfg["head_dim"])
    k_all = torch.zeros(big, dtype=W.TORCH_DTYPE[cfg["dtype"]], device=dev)
    v_all = torch.zeros(big, dtype=W.TORCH_DTYPE[cfg["dtype"]], device=dev)
    # A third case moves the most rows this tree allows: the first-level node
    # with the largest subtree is accepted alone and its whole subtree moves
    # up by the gap in front of it.
    all_layers = {}
    v_surv = W.descendants(parent, v_path[-1]) if v_path else list(range(n))
    firsts = [i for i in range(n) if parent[i] == -1]
    big_root = max(firsts, key=lambda a: len(W.descendants(parent, a)))
    cases = (("draft", v_path, v_surv), ("target", v_path, []),
             ("largest_subtree", [big_root], W.descendants(parent, big_root)))
    for side, s_path, s_surv in cases:
        s_src, _, _ = ta.kv_reroot_plan(P, cfg["capacity"], parent, s_path, s_surv)
        b = reroot_bytes(cfg, s_src, P, n_layers)
        rrot = max(1, min(P // n, math.ceil(2 * MALL_BYTES / max(b, 1)) + 1))

        def reroot_all(i, s_path=s_path, s_surv=s_surv, rrot=rrot):
            ta.kv_reroot(k_all, v_all, P - (i % rrot) * n, parent, s_path, s_surv)

        for i in range(3):
            reroot_all(i)
        _, ra_us, _ = timed(reroot_all, K, each=True)
        ra_b2b, _, _ = timed(reroot_all, K)
        ra_mean = statistics.fmean(ra_us)
        all_layers[side] = {"accepted_path": len(s_path), "survivors": len(s_surv),
                            "rows_moved": sum(1 for k, r in enumerate(s_src) if r != P + k),
                            "us_mean": round(ra_mean, 2), "us_p50": round(pct(ra_us, 50), 2),
                            "us_launch_period_back_to_back": round(ra_b2b / K, 2), "algorithmic_bytes": b,
                            "GBs": round(b / (ra_mean * 1e-6) / 1e9, 1),
                            "hbm_frac": round(b / (ra_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "rotated_positions": rrot}
    del k_all, v_all

    # One maximum-likelihood expansion step: 8 frontier leaves' draft logits
    # over the vocabulary (rotated, positively rescaled sets), 8 new nodes.
    ex_w, ex_k = 8, 8
    ex = W.make_expand_inputs(cfg, ex_w)
    e_bytes = expand_bytes(cfg, ex_w, ex_k)
    erot = max(2, math.ceil(2 * MALL_BYTES / e_bytes) + 1)
    e0 = ex["logits"].to(dev)
    e_sets = [e0 * (1.0 + 1e-3 * r) if r else e0 for r in range(erot)]
    e_scores = ex["path_scores"].to(dev)
    e_out = [torch.empty(ex_k, dtype=t, device=dev) for t in (torch.int32, torch.int32, torch.float32)]
    e_ws = torch.zeros(ta.lib().ta_tree_expand_workspace_bytes(ex_w), dtype=torch.uint8, device=dev)

    def expand(i):
        ta.tree_expand(e_sets[i % erot], e_scores, ex_k, leaf=e_out[0], token=e_out[1], score=e_out[2],
                       workspace=e_ws)

    for i in range(5):
        expand(i)
    _, ex_us, _ = timed(expand, K, each=True)
    ex_b2b, _, _ = timed(expand, K)
    _, ex_hot, _ = timed(lambda i: expand(0), 50, each=True)
    del e_sets, e0
    ex_mean = statistics.fmean(ex_us)
    ver_mean = statistics.fmean(ver_us)
    return {
        "tree_verify": {"vocab": cfg["vocab"], "rows": n + 1, "accepted_path": len(v_path),
                        "us_mean": round(ver_mean, 2), "us_p50": round(pct(ver_us, 50), 2),
                        "us_launch_period_back_to_back": round(ver_b2b / K, 2), "algorithmic_bytes": v_bytes,
                        "GBs": round(v_bytes / (ver_mean * 1e-6) / 1e9, 1),
                        "hbm_frac": round(v_bytes / (ver_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "hot_cache_us_p50": round(statistics.median(ver_hot), 2), "rotated_sets": vrot},
        "kv_reroot_all_layers": dict(layers=n_layers, **all_layers),
        "tree_expand": {"vocab": cfg["vocab"], "w": ex_w, "k": ex_k, "us_mean": round(ex_mean, 2),
                        "us_p50": round(pct(ex_us, 50), 2), "us_launch_period_back_to_back": round(ex_b2b / K, 2),
                        "hot_cache_us_p50": round(statistics.median(ex_hot), 2), "algorithmic_bytes": e_bytes,
                        "GBs": round(e_bytes / (ex_mean * 1e-6) / 1e9, 1),
                        "hbm_frac": round(e_bytes / (ex_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "rotated_sets": erot},
    }


# --------------------------------------------------------------------------
# The draft loop, run as a loop


def main_loop(args, cfg):
    """The draft-loop workload as a loop: from P = 4096, every iteration is
    one tree_attn over the current 64-node tree (one layer) and one kv_reroot
    of the cache for a random accepted path of length 1..8 and its surviving
    subtree, then the refill of the tree back to 64 nodes (new rows written
    into the cache). The refill rows, queries and plans come from the seeded
    workload, precomputed on the host. A step is one iteration; K steps run
    the iterations in order (wrapping to a fresh cache after the last).

    Each iteration's two kernels sit between their own HIP events; between
    iterations, outside those events, an untimed fill of 512 MB evicts the
    caches (in a draft step the other layers and the weights pass through
    L2 and the Infinity Cache between two uses of one layer) and the refill
    rows are copied in. value = mean over the K iterations of (tree_attn +
    kv_reroot) event time.
    """
    import torch

    import tree_masked_attention_attn_amd as ta

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    loop = W.DraftLoop(cfg)
    k0, v0 = loop.initial_cache()
    iters = []
    for _ in range(cfg["iterations"]):
        q = loop.queries()
        P, parent = loop.prefix_len, list(loop.parent)
        path, surv = loop.choose()
        src, new_par, new_p = ta.kv_reroot_plan(P, cfg["capacity"], parent, path, surv)
        keep, kr, vr = loop.advance(surv, new_par, new_p)
        c = dict(cfg, prefix=P)
        nbytes, flops, _ = tree_attn_work(c, parent)
        iters.append(dict(q=q.to(dev), P=P, parent=parent, path=path, surv=surv, new_p=new_p, keep=keep,
                          kr=kr.to(dev), vr=vr.to(dev), bytes=nbytes, flops=flops,
                          rr_bytes=reroot_bytes(cfg, src, P), splits=ta.tree_attn_num_splits(
                              k0, v0, cfg["n_q_heads"], P, cfg["n_tree"])))
    kinit, vinit = k0.to(dev), v0.to(dev)
    kd, vd = kinit.clone(), vinit.clone()
    out = torch.empty_like(iters[0]["q"])
    ws = torch.zeros(max(ta.tree_attn_workspace_bytes(kd, vd, cfg["n_q_heads"], cfg["capacity"] - 256,
                                                      cfg["n_tree"]), 1 << 20), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    n = cfg["n_tree"]
    if args.copy_calib:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def run(count, timed_events):
        ev = []
        for j in range(count):
            it = iters[j % len(iters)]
            if j % len(iters) == 0:
                kd.copy_(kinit)
                vd.copy_(vinit)
            flush.fill_(j & 255)
            e = [Ev() for _ in range(3)] if timed_events else None
            if e:
                e[0].record(stream)
            ta.tree_attn(it["q"], kd, vd, it["P"], it["parent"], out=out, workspace=ws)
            if e:
                e[1].record(stream)
            ta.kv_reroot(kd, vd, it["P"], it["parent"], it["path"], it["surv"])
            if e:
                e[2].record(stream)
                ev.append(e)
            lo, hi = it["new_p"] + it["keep"], it["new_p"] + n
            kd[:, :, lo:hi] = it["kr"]
            vd[:, :, lo:hi] = it["vr"]
        return ev

    run(args.warmup, False)
    torch.cuda.synchronize()
    K = args.steps
    wall = time.perf_counter()
    ev = run(K, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    attn_us = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
    rr_us = [e[1].elapsed_time(e[2]) * 1e3 for e in ev]
    sel = [iters[j % len(iters)] for j in range(K)]
    a_bytes = sum(it["bytes"] for it in sel)
    a_flops = sum(it["flops"] for it in sel)
    r_bytes = sum(it["rr_bytes"] for it in sel)
    a_sum, r_sum = sum(attn_us), sum(rr_us)
    hbm_gbs = a_bytes / (a_sum * 1e-6) / 1e9
    step_us = (a_sum + r_sum) / K
    roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    cpu = None
    if not args.no_cpu_baseline:
        it0 = iters[0]
        x0 = dict(q=it0["q"].cpu(), k=k0, v=v0, prefix_len=it0["P"], parent=it0["parent"], q_first=0)
        cpu = cpu_baseline(cfg, x0, it0["path"], it0["surv"], args.cpu_budget, args.cpu_budget_1t)
        cpu["sample"] += " (the loop's first iteration, P = %d)" % it0["P"]
    ps = [it["P"] for it in sel]
    line = {
        "metric": METRIC,
        "value": round(step_us, 2), "unit": "us/step", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded Gaussian q/k/v, width-8 max-likelihood tree, random accepted paths, refills)",
        "config": {"workload": cfg["name"], "mode": "loop", "iterations": len(iters),
                   "n_q_heads": cfg["n_q_heads"], "n_kv_heads": cfg["n_kv_heads"], "head_dim": cfg["head_dim"],
                   "prefix_len_first": ps[0], "prefix_len_last": ps[-1], "n_tree": n,
                   "accepted_path_mean": round(statistics.fmean(len(it["path"]) for it in sel), 2),
                   "splits": sorted({it["splits"] for it in sel})},
        "tree_attn": {"us_mean": round(a_sum / K, 2), "us_p10": round(pct(attn_us, 10), 2),
                      "us_p50": round(pct(attn_us, 50), 2), "us_p90": round(pct(attn_us, 90), 2),
                      "algorithmic_bytes_mean": round(a_bytes / K), "algorithmic_flops_mean": round(a_flops / K),
                      "hbm_GBs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4)},
        "kv_reroot": {"us_mean": round(r_sum / K, 2), "us_p50": round(pct(rr_us, 50), 2),
                      "algorithmic_bytes_mean": round(r_bytes / K),
                      "GBs": round(r_bytes / (r_sum * 1e-6) / 1e9, 2)},
        "iteration_us_p50": round(pct([a + r for a, r in zip(attn_us, rr_us)], 50), 2),
        "wall_s_timed_region": round(wall, 4),
        "kernel_source_sha": kernel_source_sha(),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


# --------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama3_70b_verify")
    ap.add_argument("--rotate", type=int, default=0, help="input sets cycled (0 = enough to exceed 2x MALL)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--cpu-budget-1t", type=float, default=6.0,
                    help="seconds of oracle work for cpu_baseline's one-thread figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true", help="also run one plain device copy (counter calibration)")
    ap.add_argument("--no-extras", action="store_true", help="skip the labelled extras (verify, expand, all layers)")
    ap.add_argument("--summarize", nargs=2, metavar=("DIR", "OUT"))
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--counters", nargs="+", metavar="OUT DIR", help="summary file, then counter-pass directories")
    ap.add_argument("--command", default=None, help="command line recorded in a summary")
    args = ap.parse_args()

    if args.summarize:
        return main_summarize(args)
    if args.traffic:
        return main_traffic(args)
    if args.counters:
        return main_counters(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the tree-attention path shards by KV head with no "
              "exchange, and this benchmark runs and reports on a single MI355X only.", file=sys.stderr)
        sys.exit(2)

    cfg = W.config(args.config)
    if cfg.get("iterations"):
        return main_loop(args, cfg)

    import torch

    import tree_masked_attention_attn_amd as ta

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = W.make_inputs(cfg, poison=False)
    parent, P = base["parent"], base["prefix_len"]
    rng = np.random.default_rng(cfg["seed"] + 1000)
    path = W.draft_path(rng, parent)
    surv = W.descendants(parent, path[-1])
    src_rows, _, _ = ta.kv_reroot_plan(P, cfg["capacity"], parent, path, surv)

    kv_set_bytes = 2 * base["k"].numel() * base["k"].element_size()
    rotate = args.rotate or max(2, math.ceil(2 * MALL_BYTES / kv_set_bytes) + 1)
    sets = []
    for r in range(rotate):
        sets.append(dict(q=base["q"].to(dev), k=(base["k"] + 0).to(dev), v=base["v"].to(dev),
                         out=torch.empty_like(base["q"], device=dev)))
        if r:  # distinct values per set (cheap perturbation on the GPU)
            sets[-1]["k"].mul_(1.0 + 1e-3 * r)
    qf = base["q_first"]
    ws_bytes = ta.tree_attn_workspace_bytes(sets[0]["k"], sets[0]["v"], cfg["n_q_heads"], P, cfg["n_tree"], qf)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calib:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def attn(i):
        s = sets[i % rotate]
        ta.tree_attn(s["q"], s["k"], s["v"], P, parent, out=s["out"], workspace=ws, q_first=qf)

    def reroot(i):
        s = sets[i % rotate]
        ta.kv_reroot(s["k"], s["v"], P, parent, path, surv)

    def step(i):
        attn(i)
        reroot(i)

    def queue_ahead(ms):
        # a device sleep so that the host enqueues everything behind it and
        # the kernels then execute back to back
        torch.cuda._sleep(int(2.4e9 * ms * 1e-3))

    def timed(fn, count, each=False):
        """Run fn(0..count-1) on the stream between two HIP events; with
        each=True also bracket every call with its own pair."""
        evs = [(Ev(), Ev())
               for _ in range(count if each else 0)]
        t0, t1 = Ev(), Ev()
        torch.cuda.synchronize()
        queue_ahead(20 * max(1, count / 200))
        wall = time.perf_counter()
        t0.record(stream)
        for i in range(count):
            if each:
                evs[i][0].record(stream)
            fn(i)
            if each:
                evs[i][1].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall
        return t0.elapsed_time(t1) * 1e3, [a.elapsed_time(b) * 1e3 for a, b in evs], wall

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back, bracketed by synchronize on
    # both sides and by HIP events on the launch stream.
    K = args.steps
    total_us, _, t_wall = timed(step, K)

    # Per-kernel figures, on the same stream and inputs: K launches of one
    # kernel, each between its own pair of events, give its average launch
    # duration (what the roofline uses; a kernel trace of the same run gives
    # the same figure to within the event packets' own cost); the same K
    # launches back to back between two events give the launch period, which
    # also holds the dispatch gap between consecutive kernels.
    _, attn_us, _ = timed(attn, K, each=True)
    attn_b2b, _, _ = timed(attn, K)
    _, reroot_us, _ = timed(reroot, K, each=True)
    rr_b2b, _, _ = timed(reroot, K)
    # One input set only (L2 / Infinity Cache warm), labelled as such.
    _, hot, _ = timed(lambda i: attn(0), 50, each=True)
    hot_us = statistics.median(hot)

    extras = {} if args.no_extras else run_extras(ta, torch, cfg, dev, parent, P, K, timed)


    nbytes, flops, anc = tree_attn_work(cfg, parent)
    splits = ta.tree_attn_num_splits(sets[0]["k"], sets[0]["v"], cfg["n_q_heads"], P, cfg["n_tree"], qf)
    block_rows = ta.tree_attn_block_rows(sets[0]["k"], sets[0]["v"], cfg["n_q_heads"], P, cfg["n_tree"], qf)
    rr_bytes = reroot_bytes(cfg, src_rows, P)
    attn_mean = statistics.fmean(attn_us)
    rr_mean = statistics.fmean(reroot_us)
    hbm_gbs = nbytes / (attn_mean * 1e-6) / 1e9
    tflops = flops / (attn_mean * 1e-6) / 1e12
    traffic = load_traffic(cfg)
    if cfg["dtype"] == "bf16" and flops / BF16_PEAK_TFLOPS > nbytes / HBM_PEAK_GBS * 1e3:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, base, path, surv, args.cpu_budget, args.cpu_budget_1t)

    step_us = total_us / K
    line = {
        "metric": METRIC,
        "value": round(step_us, 2),
        "unit": "us/step",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (seeded Gaussian q/k/v, width-8 max-likelihood tree)",
        "config": {"workload": cfg["name"], "n_q_heads": cfg["n_q_heads"], "n_kv_heads": cfg["n_kv_heads"],
                   "head_dim": cfg["head_dim"], "prefix_len": P, "n_tree": cfg["n_tree"], "q_first": qf,
                   "visible_tree_pairs": anc, "accepted_path": len(path), "survivors": len(surv),
                   "rotated_sets": rotate, "splits": splits, "block_rows": block_rows},
        "tree_attn": {"us_mean": round(attn_mean, 2), "us_p10": round(pct(attn_us, 10), 2),
                      "us_p50": round(pct(attn_us, 50), 2), "us_p90": round(pct(attn_us, 90), 2),
                      "us_launch_period_back_to_back": round(attn_b2b / K, 2),
                      "hot_cache_us_p50": round(hot_us, 2),
                      "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                      "split_partial_bytes_written": split_partial_bytes(cfg, splits, block_rows),
                      "split_partial_bytes_read": split_partial_bytes(cfg, splits, block_rows),
                      "hbm_GBs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                      "TFLOPs": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
        "kv_reroot": {"us_mean": round(rr_mean, 2), "us_p50": round(pct(reroot_us, 50), 2),
                      "us_launch_period_back_to_back": round(rr_b2b / K, 2),
                      "algorithmic_bytes": rr_bytes, "GBs": round(rr_bytes / (rr_mean * 1e-6) / 1e9, 2)},
        **extras,
        "wall_s_timed_region": round(t_wall, 4),
        "kernel_source_sha": kernel_source_sha(),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
