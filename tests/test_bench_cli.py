"""The benchmark's command line and result-line helpers, without a GPU: more
than one GPU is refused with a message and exit status 2 (this build measures
one GPU); the counter summary mode turns two rocprofv3 counter files into the
calibrated per-launch HBM figure, which the result line carries only for the
workload and kernel build it was taken on; the tree shapes it reports come
from the parent arrays; the roofline's algorithmic flops and bytes match the
headline workload's closed form and a pair-by-pair count of visible keys."""
import csv
import json
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they
    read for the 1 GiB calibration copy; the attention figure is the mean over
    its dispatches."""
    sys.path.insert(0, ROOT)
    import bench
    attn = "void sv::" + bench.ATTN_KERNEL + "<128, 3, 4>(sv::AttnParams)"
    copy = "void at::native::" + bench.COPY_KERNEL + "_x(float)"   # a name containing the copy kernel's
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # the 1 GiB copy: FETCH_SIZE shows half of its 2^20 KiB, WRITE_SIZE all of it
    _counter_csv(fetch, "FETCH_SIZE", [(attn, 500000.0), (attn, 520000.0), (copy, 524288.0)])
    _counter_csv(write, "WRITE_SIZE", [(attn, 30000.0), (attn, 34000.0), (copy, 1048576.0)])
    out = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS", str(out))
    bench.summarize_counters(str(fetch), str(write))
    d = json.loads(out.read_text())
    assert abs(d["fetch_scale"] - 2.0) < 1e-9 and abs(d["write_scale"] - 1.0) < 1e-9
    want = 1024 * (510000.0 * 2.0 + 32000.0 * 1.0)
    assert abs(d["hbm_bytes_per_launch"] - want) < 1.0


def test_counter_hash_tracks_flags_not_location(monkeypatch):
    """The counter summary is keyed by the attention source and its compiler
    flags: another flag changes the key, another checkout location does not."""
    import bench
    from eagle_tree_verification_attn_amd import build as B
    h0 = bench.attn_build_hash()
    moved = [("/elsewhere/include" if os.sep in f else f) for f in B.CFLAGS]
    monkeypatch.setattr(B, "CFLAGS", moved)
    assert bench.attn_build_hash() == h0
    monkeypatch.setattr(B, "FILE_FLAGS", {"attn.hip": B.FILE_FLAGS["attn.hip"] + ["-O2"]})
    assert bench.attn_build_hash() != h0


def test_counter_traffic_only_for_its_workload(tmp_path, monkeypatch):
    """The committed counters are taken on the default workload: the result
    line carries their HBM bytes for that workload only (null for any other
    --config), and only while the kernel's source and flags are unchanged."""
    import bench
    out = tmp_path / "counters.json"
    out.write_text(json.dumps({"attn_build_sha256": bench.attn_build_hash(), "hbm_bytes_per_launch": 123456}))
    monkeypatch.setattr(bench, "COUNTERS", str(out))
    assert bench.counters_traffic(bench.WORKLOAD) == 123456.0
    assert bench.counters_traffic("long_ctx_dynamic") is None
    out.write_text(json.dumps({"attn_build_sha256": "0" * 64, "hbm_bytes_per_launch": 123456}))
    assert bench.counters_traffic(bench.WORKLOAD) is None


def test_tree_shape_of_the_result_line():
    """Drafted nodes (root excluded) and depth per sequence, from the parent
    arrays: one number when all sequences agree, else one per sequence."""
    import types
    import numpy as np
    import bench
    chain = [-1, 0, 1, 2, -1]          # root, then a chain of 3 (depth 3); one unused slot
    star = [-1, 0, 0, 0, 0]            # root with 4 children (depth 1)
    inst = types.SimpleNamespace(B=2, num_nodes=np.array([4, 5]), parent=np.array([chain, star]))
    assert bench.tree_shape(inst) == ([3, 4], [3, 1])
    same = types.SimpleNamespace(B=2, num_nodes=np.array([5, 5]), parent=np.array([star, star]))
    assert bench.tree_shape(same) == (4, 1)


def test_kv_head_shard_is_one_gpus_share():
    """`bench.py --kv-shards n` times one GPU's share under an n-way KV-head
    split: Hq / n and Hkv / n heads, everything else as in the workload; a
    split that does not divide the KV heads is refused."""
    import pytest
    from synth import config_by_name, kv_head_shard
    full = config_by_name("tree64_llama70b_b32")
    s = kv_head_shard("tree64_llama70b_b32", 8)
    assert (s["Hq"], s["Hkv"]) == (8, 1) and s["Hq"] // s["Hkv"] == full["Hq"] // full["Hkv"]
    assert {k: v for k, v in s.items() if k not in ("Hq", "Hkv", "name")} == \
        {k: v for k, v in full.items() if k not in ("Hq", "Hkv", "name")}
    assert s["name"] != full["name"]
    assert kv_head_shard(full, 1) == full
    with pytest.raises(ValueError):
        kv_head_shard(full, 3)


def _tree_from_widths(widths):
    """Parent array of a tree numbered by depth: each node's parent is the
    first node of the previous depth (depth sums do not depend on which)."""
    parent = [-1]
    first_prev, n = 0, 1
    for w in widths:
        parent += [first_prev] * w
        first_prev, n = n, n + w
    return np.array(parent, dtype=np.int64)


def test_algorithmic_work_of_the_headline_workload():
    """The roofline's numerator and byte count for 32 sequences, 64/8 heads,
    head dim 128, prefix 8192 and the 65-position tree of widths
    4/8/12/12/14/14: positions at depth d see d + 1 tree keys, so the tree
    adds 1*1 + 4*2 + 8*3 + 12*4 + 12*5 + 14*6 + 14*7 = 323 visible pairs per
    query head and sequence."""
    import bench
    B, Hq, Hkv, D, L, T = 32, 64, 8, 128, 8192, 65
    parent = np.tile(_tree_from_widths([4, 8, 12, 12, 14, 14]), (B, 1))
    inst = types.SimpleNamespace(B=B, Hq=Hq, Hkv=Hkv, D=D, T_max=T, dtype="bf16", parent=parent,
                                 num_nodes=np.full(B, T), prefix_len=np.full(B, L))
    flops, nbytes = bench.algorithmic_work(inst)
    assert flops == 4 * Hq * D * B * (T * L + 323) == 558_684_438_528
    # bf16: prefix K and V once, Q in and O out, the tree's K and V, one mask word per position
    assert nbytes == 2 * (2 * B * Hkv * L * D + 2 * B * T * Hq * D + 2 * B * T * Hkv * D) + 8 * B * T * 2
    assert nbytes == 1_150_452_224


def test_algorithmic_work_counts_visible_pairs():
    """Ragged sequences: the flop count is 4 * D per (query head, visible key)
    pair, counted here pair by pair from the ancestor sets."""
    import bench
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, T = 3, 4, 2, 64, 9
    parent = np.full((B, T), -1, dtype=np.int64)
    num_nodes = np.array([9, 1, 5])
    for b in range(B):
        for i in range(1, int(num_nodes[b])):
            parent[b, i] = rng.integers(0, i)
    prefix = np.array([100, 0, 7])
    inst = types.SimpleNamespace(B=B, Hq=Hq, Hkv=Hkv, D=D, T_max=T, dtype="f32", parent=parent,
                                 num_nodes=num_nodes, prefix_len=prefix)
    pairs = 0
    for b in range(B):
        for i in range(int(num_nodes[b])):
            seen, j = 0, i
            while j >= 0:          # the node and its ancestors
                seen += 1
                j = int(parent[b, j])
            pairs += int(prefix[b]) + seen
    flops, _ = bench.algorithmic_work(inst)
    assert flops == 4 * Hq * D * pairs
