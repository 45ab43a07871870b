"""bench.py on the CPU: the one-GPU contract, the algorithmic work counts and
the rocprofv3 summary tools (on synthetic profiler output). No GPU needed."""

import csv
import ctypes
import json
import os
import sqlite3
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import tree_masked_attention_attn_amd as ta  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["llama3_70b_verify", "llama3_70b_verify_bs8", "draft_expand_w8", "tiny_fp32"])
def test_tree_attn_work_counts_visible_pairs_and_bytes(name):
    cfg = W.config(name)
    parent, _ = W.make_tree(cfg, np.random.default_rng(cfg["seed"]))
    nbytes, flops, anc = bench.tree_attn_work(cfg, parent)
    qf, n = cfg.get("q_first", 0), cfg["n_tree"]
    want_anc = sum(len(oracle.ancestors_inclusive(parent, i)) for i in range(qf, n))
    assert anc == want_anc
    es = 4 if cfg["dtype"] == "f32" else 2
    P, d, hq, hkv = cfg["prefix"], cfg["head_dim"], cfg["n_q_heads"], cfg["n_kv_heads"]
    # every visible (row, key) pair: the whole prefix plus the root path, QK and PV
    assert flops == 4 * d * hq * sum(P + len(oracle.ancestors_inclusive(parent, i)) for i in range(qf, n))
    assert nbytes == 2 * hkv * d * es * (P + n) + 2 * (n - qf) * hq * d * es + 4 * n
    if name == "llama3_70b_verify":
        assert (nbytes, flops) == (35_913_984, 17_189_306_368)


def test_reroot_verify_expand_byte_counts():
    cfg = W.config("llama3_70b_verify")
    # rows already in place move nothing
    assert bench.reroot_bytes(cfg, [8192, 8193], 8192, n_layers=80) == 0
    # one moved row: read + write, K and V, every KV head and layer
    assert bench.reroot_bytes(cfg, [8195], 8192, n_layers=80) == 2 * 2 * 8 * 128 * 2 * 80
    assert bench.verify_bytes(cfg, 64) == 65 * 128256 * 2 + 4 * 64 + 4 * 65 + 4 * 66
    assert bench.expand_bytes(cfg, 8, 8) == 8 * 128256 * 2 + 4 * 8 + 12 * 8


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_summary_of_kernel_stats_and_of_a_rocpd_database(tmp_path):
    d = tmp_path / "stats"
    d.mkdir()
    _write_csv(d / "run_kernel_stats.csv", [
        {"Name": "tree_attn_bf16_kernel<128, 1>", "Calls": 10, "TotalDurationNs": 300000, "AverageNs": 30000,
         "MinNs": 29000, "MaxNs": 31000, "Percentage": 90.0}])
    lines, _ = bench.summarize(str(d), "x.md", "cmd")
    assert any("tree_attn_bf16_kernel" in l and "| 10 | 300.0 | 30.00 | 29.00 | 31.00 |" in l for l in lines)
    db_dir = tmp_path / "db"
    db_dir.mkdir()
    con = sqlite3.connect(str(db_dir / "run_results.db"))
    con.execute("create table kernels (name text, duration integer)")
    con.executemany("insert into kernels values (?, ?)", [("tree_verify_kernel", 7000), ("tree_verify_kernel", 9000)])
    con.commit()
    con.close()
    lines, _ = bench.summarize(str(db_dir), "y.md", "cmd")
    assert any("tree_verify_kernel | 2 | 16.0 | 8.00 | 7.00 | 9.00 |" in l for l in lines)


def test_traffic_record_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    def counters(path, name, attn_kib, copy_kib):
        path.mkdir()
        rows = [{"Kernel_Name": "tree_attn_bf16_kernel", "Counter_Name": name, "Dispatch_Id": i,
                 "Counter_Value": attn_kib} for i in range(3)]
        rows += [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": name, "Dispatch_Id": 10,
                  "Counter_Value": copy_kib},
                 {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": name, "Dispatch_Id": 11,
                  "Counter_Value": 4.0}]  # a small upload: not the calibration copy
        _write_csv(path / "run_counter_collection.csv", rows)

    copy_kib = bench.COPY_BYTES / 1024
    counters(tmp_path / "fetch", "FETCH_SIZE", 1000.0, copy_kib / 2)  # FETCH counts half the bytes
    counters(tmp_path / "write", "WRITE_SIZE", 300.0, copy_kib)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    args = type("A", (), {"traffic": (str(tmp_path / "fetch"), str(tmp_path / "write")),
                          "config": "llama3_70b_verify", "command": "cmd"})()
    bench.main_traffic(args)
    text = open(bench.traffic_file(W.config("llama3_70b_verify"))).read()
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    assert rec["copy_fetch_factor"] == 0.5 and rec["copy_write_factor"] == 1.0
    assert rec["traffic_bytes"] == int((1000.0 / 0.5 + 300.0) * 1024)
    assert rec["source_sha"] == bench.kernel_source_sha()
    assert bench.load_traffic(W.config("llama3_70b_verify")) == rec["traffic_bytes"]


def test_split_partial_bytes_match_the_traffic_excess_model():
    cfg = W.config("llama3_70b_verify")
    # 8 KV heads x 4 row blocks x 8 splits = 256 units of 128 rows, fp32 O + fp32 (max, sum)
    assert bench.split_partial_bytes(cfg, 8, 128) == 256 * 128 * (8 + 128 * 4)
    assert bench.split_partial_bytes(cfg, 1, 128) == 0
    tiny = W.config("tiny_fp32")
    assert bench.split_partial_bytes(tiny, 2, 128) == 1 * 1 * 2 * 128 * (8 + 64 * 4)
    # bs = 8 verify: one 64-row block per KV head, both of its tiles written
    bs8 = W.config("llama3_70b_verify_bs8")
    assert bench.split_partial_bytes(bs8, 16, 64) == 8 * 16 * 64 * (8 + 128 * 4)
    # 8B verify in 64-row blocks: 8 KV heads x 4 blocks x 8 splits = 256 units of 64 rows
    assert bench.split_partial_bytes(W.config("llama3_8b_verify"), 8, 64) == 256 * 64 * (8 + 128 * 4)
    # 300 rows per KV head in 64-row blocks: the last block's 44 rows take two 32-row tiles
    ragged = dict(n_q_heads=12, n_kv_heads=4, head_dim=128, dtype="bf16", n_tree=100)
    assert bench.split_partial_bytes(ragged, 4, 64) == 4 * 4 * (4 * 64 + 64) * (8 + 128 * 4)


@pytest.mark.parametrize("name", ["llama3_70b_verify", "qwen2_72b_32k_verify", "llama3_8b_verify",
                                  "llama3_70b_verify_bs8"])
def test_committed_traffic_is_the_algorithmic_bytes_plus_the_partials_both_ways(name):
    """The FETCH_SIZE/WRITE_SIZE records in profiles/ against the traffic
    model: q, out and every K/V byte once, the split partials written once
    and read back once (within 5%). These shapes keep each KV head's row
    blocks on one XCD; the TP = 4 share, whose heads span four XCDs, fetches
    its K/V once per XCD and is not one of them."""
    cfg = W.config(name)
    path = bench.traffic_file(cfg)
    if not os.path.exists(path):
        pytest.skip(f"no traffic record for {name}")
    with open(path) as f:
        rec = json.loads(f.read().split("```json", 1)[1].split("```", 1)[0])
    parent, _ = W.make_tree(cfg, np.random.default_rng(cfg["seed"]))
    nbytes, _, _ = bench.tree_attn_work(cfg, parent)
    es = 2 if cfg["dtype"] == "bf16" else 4
    desc = ta.ta_kv_cache(1 << 40, 1 << 41, 1, cfg["n_kv_heads"], cfg["capacity"], cfg["head_dim"],
                          ta.TA_BF16 if es == 2 else ta.TA_F32)
    qf = cfg.get("q_first", 0)
    lib = ta.lib()
    splits = lib.ta_tree_attn_rows_num_splits(ctypes.byref(desc), cfg["n_q_heads"], cfg["prefix"], cfg["n_tree"], qf)
    block = lib.ta_tree_attn_rows_block_rows(ctypes.byref(desc), cfg["n_q_heads"], cfg["prefix"], cfg["n_tree"], qf)
    model = nbytes + 2 * bench.split_partial_bytes(cfg, splits, block)
    assert abs(rec["traffic_bytes"] - model) <= 0.05 * model, (rec["traffic_bytes"], model)


def test_counter_summary_derives_rocprof_utilisations(tmp_path):
    # two counter passes of 2 dispatches each; GRBM_GUI_ACTIVE comes once per XCD (summed by the CSV)
    agent = [{"Name": "gfx950", "Num_Xcc": 8, "Cu_Count": 256, "Simd_Count": 1024}]

    def counter_pass(name, values):
        d = tmp_path / name
        d.mkdir()
        _write_csv(d / "run_agent_info.csv", agent)
        rows = [{"Kernel_Name": "tree_attn_bf16_kernel<128, 1>", "Counter_Name": c, "Dispatch_Id": i,
                 "Counter_Value": v} for i in range(2) for c, v in values.items()]
        _write_csv(d / "run_counter_collection.csv", rows)
        return str(d)

    gui = 8 * 50_000.0  # 50k cycles per XCD
    p1 = counter_pass("p1", {"GRBM_GUI_ACTIVE": gui, "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 50_000 * 1024})
    p2 = counter_pass("p2", {"GRBM_GUI_ACTIVE": gui, "SQ_INSTS_MFMA": 0.25 * 50_000 * 1024 / 32,
                             "SQ_LDS_IDX_ACTIVE": 0.1 * 50_000 * 256, "SQ_LDS_BANK_CONFLICT": 0.0,
                             "SQ_INSTS_VALU": 9 * 0.25 * 50_000 * 1024 / 32})
    lines, means, derived = bench.counter_summary([p1, p2], "cmd", "llama3_70b_verify")
    assert lines[0] == "# rocprofv3 counters: tree_attn, llama3_70b_verify"
    assert means["GRBM_GUI_ACTIVE"] == gui
    assert abs(derived["MfmaUtil (% of SIMD cycles, GPU-active basis)"] - 25.0) < 1e-9
    assert derived["MFMA busy cycles per MFMA instruction"] == 32.0
    assert abs(derived["LDS indexed-access utilisation (% of CU cycles, GPU-active basis)"] - 10.0) < 1e-9
    assert derived["LDS bank-conflict cycles per conflict-free LDS cycle"] == 0.0
    assert derived["VALU instructions per MFMA instruction"] == 9.0
