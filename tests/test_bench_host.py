"""Host-side logic of bench.py (CPU only): the algorithmic byte count behind
the roofline figure, the HBM traffic record written from rocprofv3 counter
CSVs and the source-hash gate that retires it, and the one-GPU contract."""
import csv
import json
import os
import subprocess
import sys

import numpy as np

import bench
from synth import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_by_item():
    """The verify bytes counted item by item: every (sequence, head) reads its
    context's K and V rows, every real node reads q, k_new and v_new rows and
    writes its out row, plus block-table entries (one int32 per started
    page), two int32 tree entries per real node and one (cos, sin) row of
    d/2 float pairs per distinct depth."""
    wl = make_workload("vicuna7b_b16", 3, batch=3, heads=2, ctx_range=(1, 300))
    s = wl.spec
    es = 2  # bf16
    total = 0
    for b in range(s.batch):
        ctx, t = int(wl.ctx_lens[b]), int(wl.tree_sizes[b])
        for _h in range(s.kv_heads):
            total += ctx * 2 * s.head_dim * es            # cached K and V rows
            total += t * 2 * s.head_dim * es              # k_new and v_new rows
        for _h in range(s.heads):
            total += t * 2 * s.head_dim * es              # q rows read, out rows written
        total += -(-ctx // 16) * 4                        # page ids
        total += t * 2 * 4                                # parent and depth
        depths = {int(x) for x in wl.tree_depth[b, :t]}
        total += len(depths) * (s.head_dim // 2) * 2 * 4  # one (cos, sin) row per depth
    got = bench.algorithmic_bytes(wl)
    assert got["verify"] == total
    assert got["commit"] == 0
    L = np.array([1, 3, 2])
    rows = int((L * 2 * s.kv_heads * s.head_dim * es * 2).sum())  # read k/v_new, write pages
    assert bench.algorithmic_bytes(wl, L)["commit"] == rows


def test_algorithmic_bytes_of_the_benchmarked_workload():
    """The figure the roofline is quoted on (7B-shaped batch 16, seed 0)."""
    wl = make_workload("vicuna7b_b16", 0)
    got = bench.algorithmic_bytes(wl)
    assert got["verify"] == 345_772_736
    assert got["kv"] == int((wl.ctx_lens.astype(np.int64) * 2 * 32 * 128 * 2).sum())


def _counter_csv(path, counter, verify_kb, copy_kb):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in verify_kb:
            w.writerow({"Kernel_Name": "ta::(anonymous namespace)::verify_mfma_kernel(ta::VerifyParams)",
                        "Counter_Name": counter, "Counter_Value": v})
        for v in copy_kb:
            w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                        "Counter_Value": v})
        w.writerow({"Kernel_Name": "vocab_argmax_kernel", "Counter_Name": counter,
                    "Counter_Value": 123.0})


def test_traffic_record_and_its_gate(tmp_path, monkeypatch):
    """Per-dispatch means of the verify kernel, each counter scaled by what it
    reads for the 512 MiB copies (the five largest copy dispatches); the
    record is reported only for its workload and kernel, and only while the
    kernel sources hash to the recorded value."""
    copy_kb = (512 << 20) / 1024
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them
    _counter_csv(fetch, "FETCH_SIZE", [1000.0, 1200.0], [7.0] + [copy_kb / 2] * 5)
    _counter_csv(write, "WRITE_SIZE", [50.0, 70.0], [3.0] + [copy_kb] * 5)
    record = tmp_path / "record.json"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(record))
    bench.write_traffic_record(str(fetch), str(write), "vicuna7b_b16", 0)
    rec = json.load(open(record))
    assert rec["dispatches"] == [2, 2]
    assert rec["copy_calibration"]["fetch_scale"] == 2.0
    assert rec["copy_calibration"]["write_scale"] == 1.0
    assert rec["traffic_bytes_per_launch"] == int((1100.0 * 2 + 60.0) * 1024)
    assert bench.counted_traffic("vicuna7b_b16", "verify_mfma_kernel") == \
        rec["traffic_bytes_per_launch"]
    assert bench.counted_traffic("vicuna13b_b8", "verify_mfma_kernel") is None
    assert bench.counted_traffic("vicuna7b_b16", "verify_stream_kernel") is None
    rec["sources_sha256"] = "0" * 64            # as if a kernel source had changed
    json.dump(rec, open(record, "w"))
    assert bench.counted_traffic("vicuna7b_b16", "verify_mfma_kernel") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_full_binary_preset_takes_larger_tree_sizes():
    """The preset built on a fixed full binary tree grows the tree to a
    requested size: every sequence's real nodes are a prefix of a full binary
    tree in BFS order (node i's parent is (i - 1) // 2), as many as drawn."""
    wl = make_workload("tiny", 4, batch=6, heads=1, tree_sizes=(1, 5, 26, 63))
    assert wl.spec.t_max == 63
    for b in range(6):
        par = np.asarray(wl.tree_parent[b])
        n = int(np.sum(par != -2))
        assert n in (1, 5, 26, 63)
        assert par[0] == -1 and all(par[i] == (i - 1) // 2 for i in range(1, n))
        assert np.all(par[n:] == -2)
