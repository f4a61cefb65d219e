"""The benchmark's command line, without a GPU: more than one GPU is refused
with a message and exit status 2 (this build measures one GPU), and the
counter summary mode turns two rocprofv3 counter files into the calibrated
per-launch HBM figure."""
import csv
import json
import os
import subprocess
import sys

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
