"""Host-side logic of bench.py, no GPU: the kernel-trace summary (per-dispatch
distribution, and the per-call span of two-launch calls), the algorithmic byte
count against a hand count, and the refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from workloads import make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)


def test_summarize_trace_one_launch(tmp_path):
    rows, t = [], 1000
    durs = [10.0 + i for i in range(11)]            # 10 .. 20 us
    for d in durs:
        rows.append({"Kernel_Name": "spin_kernel", "Start_Timestamp": t, "End_Timestamp": t + 500})
        t += 600
        rows.append({"Kernel_Name": "void ta::attn_kernel<...>(ta::Params)",
                     "Start_Timestamp": t, "End_Timestamp": t + int(d * 1000)})
        t += int(d * 1000) + 700
    p = tmp_path / "trace.csv"
    _write_trace(p, rows)
    s = bench.summarize_trace(str(p), "attn_kernel")
    assert s["dispatches"] == 11
    assert s["median_us"] == 15.0 and s["min_us"] == 10.0 and s["max_us"] == 20.0
    assert s["mean_us"] == 15.0
    assert s["p10_us"] == pytest.approx(11.0) and s["p90_us"] == pytest.approx(19.0)
    assert "call_span" not in s                      # no combine launches


def test_summarize_trace_two_launches(tmp_path):
    # attention, then combine, per call; a gap between them and between calls;
    # rows deliberately out of order in the file
    rows, t = [], 0
    for i in range(10):
        a0, a1 = t, t + 12000 + 100 * i
        c0, c1 = a1 + 1500, a1 + 1500 + 4000
        rows.append({"Kernel_Name": "ta::combine_kernel<...>", "Start_Timestamp": c0, "End_Timestamp": c1})
        rows.append({"Kernel_Name": "ta::attn_kernel<...>", "Start_Timestamp": a0, "End_Timestamp": a1})
        t = c1 + 2000
    p = tmp_path / "trace2.csv"
    _write_trace(p, rows)
    s = bench.summarize_trace(str(p), "attn_kernel")
    assert s["dispatches"] == 10
    assert s["combine_kernel"]["dispatches"] == 10 and s["combine_kernel"]["median_us"] == 4.0
    spans = sorted(12.0 + 0.1 * i + 1.5 + 4.0 for i in range(10))
    assert s["call_span"]["min_us"] == pytest.approx(spans[0])
    assert s["call_span"]["max_us"] == pytest.approx(spans[-1])


def test_algorithmic_bytes_hand_count():
    # one sequence, 2 KV heads, D = 16, bf16, prefix 70 tokens, a 3-node tree:
    # K and V of 70 tokens x 2 heads x 16 x 2 B, the tree's K and V
    # (3 x 2 x 16 x 2 B each), q and out (3 x 4 heads x 16 x 2 B each),
    # lse (3 x 4 x 4 B), and the int32 metadata (block ids, prefix length,
    # parents, tree offset)
    rng = np.random.default_rng(0)
    inp = make_inputs(dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=16,
                      prefix_lens=[70], trees=[[-1, 0, 0]], rng=rng)
    kv = 2 * 70 * 2 * 16 * 2
    tree_kv = 2 * 3 * 2 * 16 * 2
    q_out = 2 * 3 * 4 * 16 * 2
    lse = 3 * 4 * 4
    got = bench.algorithmic_bytes(inp)
    assert got >= kv + tree_kv + q_out + lse
    meta = got - (kv + tree_kv + q_out + lse)
    # block table (2 blocks), prefix length, 3 parents and one tree offset
    # per sequence (B + 1 offsets for B sequences, counted as B)
    assert meta == 4 * (2 + 1 + 3 + 1)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
