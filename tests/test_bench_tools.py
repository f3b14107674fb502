"""The benchmark's measurement tooling on the CPU: the algorithmic byte and
FLOP counts it divides by, the rocprofv3 counter and traffic summaries it
writes into profiles/, and its refusal of more than one GPU."""

import csv
import json
import os
import subprocess
import sys

import numpy as np

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_bytes_count_each_context_once():
    # K and V rows of every cached token, q in and out, table entries, lengths
    c = wl.make_case("b", "decode", 1, [1, 256, 257], 16, 8)
    ctx = 1 + 256 + 257
    want = ctx * 8 * 128 * 2 * 2 + 2 * 3 * 16 * 128 * 2 + 4 * (1 + 1 + 2) + 4 * 3
    assert bench.decode_bytes(c) == want


def test_prefill_flops_count_visible_pairs_only():
    # causal, prompt only: row i sees i + 1 keys; with a cached prefix of p
    # tokens, row i sees p + i + 1 keys
    c = wl.make_case("p", "prefill", 2, [5, 7], 16, 8, q_lens=[5, 3])
    pairs = sum(i + 1 for i in range(5)) + sum(4 + i + 1 for i in range(3))
    assert bench.prefill_flops(c) == 4 * 128 * 16 * pairs


def test_prefill_bytes_count_q_out_and_each_context_once():
    # q rows in and out (every head), K and V rows of every context once,
    # table entries of the contexts, lengths and the query offsets
    c = wl.make_case("pb", "prefill", 3, [5, 300], 16, 8, q_lens=[5, 3])
    want = 2 * (5 + 3) * 16 * 128 * 2 + (5 + 300) * 8 * 128 * 2 * 2 + 4 * (1 + 2) + 4 * 2 + 4 * 3
    assert bench.prefill_bytes(c) == want


def test_committed_prefill_traffic_summary_is_current_and_plausible():
    """The prefill traffic summary records the current prefill sources; its
    writes are the output rows exactly (each written once) and its reads lie
    between the algorithmic reads (q, every K/V row once) and a few times
    them (K/V rows re-fetched after L2 eviction)."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "prefill_8x2048_traffic.json")))
    assert rec["source_sha256_16"] == bench.prefill_digest()
    c = wl.prefill_8x2048()
    out_bytes = int(c.q_lens.sum()) * c.num_q_heads * c.head_dim * 2
    assert abs(rec["write_bytes"] - out_bytes) <= 0.01 * out_bytes
    reads = bench.prefill_bytes(c) - out_bytes
    assert reads <= rec["fetch_bytes"] < 4 * reads


def _write_counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_averages_dispatches_and_derives_mfma_busy(tmp_path):
    k = "void pa::prefill_kernel<2>(pa::PrefillArgs)"
    p1 = tmp_path / "p1.csv"
    _write_counter_csv(p1, [
        {"Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 1000.0},
        {"Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 3000.0},
        {"Kernel_Name": k, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 80.0},
        {"Kernel_Name": k, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 80.0},
        {"Kernel_Name": "other", "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1e9},
    ])
    out = tmp_path / "s.md"
    res = bench.summarize_counters(str(out), "prefill_kernel<2>", [str(p1)], ["cmd"])
    assert res["counters"]["SQ_VALU_MFMA_BUSY_CYCLES"] == 2000.0
    # busy / (1024 SIMDs x GRBM cycles per XCD (80 / 8))
    assert abs(res["ratios"]["mfma_busy_frac"] - 2000.0 / (1024 * 10.0)) < 1e-12
    assert out.exists() and (tmp_path / "s.json").exists()
    assert json.load(open(tmp_path / "s.json"))["commands"] == ["cmd"]


def test_traffic_summary_scales_by_the_copy_of_known_size(tmp_path):
    k = "void pa::decode_split_kernel<2, false, true>(pa::DecodeArgs)"
    copy = "__amd_rocclr_copyBuffer"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy of 1 MiB reads as 512 KiB fetched and 1024 KiB written
    _write_counter_csv(f, [{"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
                           {"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
                           {"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 512.0}])
    _write_counter_csv(w, [{"Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0},
                           {"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024.0}])
    res = bench.summarize_traffic(str(f), str(w), 1, "decode_split_kernel<2, false, true>",
                                  str(tmp_path / "t.json"), ["a", "b"])
    assert res["dispatches"] == 2
    assert abs(res["fetch_scale"] - 2.0) < 1e-12 and abs(res["write_scale"] - 1.0) < 1e-12
    assert res["fetch_bytes"] == 200.0 * 1024 * 2.0
    assert res["write_bytes"] == 10.0 * 1024
    assert res["traffic_bytes"] == res["fetch_bytes"] + res["write_bytes"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_committed_traffic_summaries_match_their_algorithmic_bytes():
    """The committed decode traffic summaries read within a few per cent of
    the algorithmic bytes of the same workload (no re-reads)."""
    for name in ("qwen3_0.6b_decode", "qwen3_4b_decode", "long_context_decode"):
        path = os.path.join(ROOT, "profiles", f"decode_{name}_traffic.json")
        if not os.path.exists(path):
            continue
        rec = json.load(open(path))
        alg = bench.append_bytes(wl.CONFIGS[name]())
        assert 0.99 < rec["traffic_bytes"] / alg < 1.05, (name, rec["traffic_bytes"], alg)
    assert np.isfinite(bench.HBM_PEAK_GBS)
