#!/usr/bin/env python3
"""Tree-verification benchmark on one MI355X.

One step = sv_verify_step (tree mask -> tree attention -> per-node target
softmax statistics -> accept / reject walk) over one batch of the
Llama-3-70B-shaped workload: 32 sequences, 64 query / 8 KV heads, head dim 128,
KV prefix 8192, a 64-node draft tree of depth 6, vocabulary 128256,
temperature 0.8, bf16.  Inputs are synthetic (seeded), generated on the host
and resident in HBM before timing starts.

Prints one JSON line: steps/s, ms per step, per-kernel times (HIP events on
the launch stream), the roofline of the dominant kernel, and the CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 200] [--warmup 10] [--prewarm-seconds 2]
    python bench.py --kernels-only   (for rocprofv3 runs: kernels + a copy of known size)
    python bench.py --summarize-counters FETCH.csv WRITE.csv
        (turns two rocprofv3 --pmc runs of --kernels-only, FETCH_SIZE then
         WRITE_SIZE, into the per-launch HBM traffic summary of the attention
         kernel, calibrated against the 1 GiB copy)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify steps/sec (attn+accept) and % HBM roofline, B=32 70B-shape"
WORKLOAD = "tree64_llama70b_b32"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
COUNTERS = os.path.join(ROOT, "profiles", "tree_attn_tree64_llama70b_b32_counters.json")
COPY_BYTES = 1 << 30            # the calibration copy of --kernels-only (read once, written once)
ATTN_KERNEL = "k_attn_bf16"
COPY_KERNEL = "neg_kernel"
ATTN_SRC = os.path.join(ROOT, "eagle_tree_verification_attn_amd", "csrc", "attn.hip")


def tree_depths(parent, num_nodes):
    """Depth of every node (root 0) from the parent arrays (parents precede children)."""
    import numpy as np
    depth = np.zeros(parent.shape, dtype=np.int64)
    for b in range(parent.shape[0]):
        for i in range(1, int(num_nodes[b])):
            depth[b, i] = depth[b, int(parent[b, i])] + 1
    return depth


def algorithmic_work(inst):
    """Algorithmic attention flops and bytes of one step.

    4 * D flops per (query head, visible key) pair -- QK^T and PV -- over L_b
    prefix keys plus depth+1 ancestor keys per position; bytes = the prefix K
    and V once, Q in, O out, tree K/V once, mask words.
    """
    s = 2 if inst.dtype == "bf16" else 4
    depth = tree_depths(inst.parent, inst.num_nodes)
    pairs = 0
    for b in range(inst.B):
        T = int(inst.num_nodes[b])
        pairs += T * int(inst.prefix_len[b]) + int((depth[b, :T] + 1).sum())
    flops = 4.0 * inst.Hq * inst.D * pairs
    W = (inst.T_max + 63) // 64
    attn_bytes = float(s * (2 * inst.Hkv * inst.D * int(inst.prefix_len.sum())
                            + 2 * inst.Hq * inst.D * int(inst.num_nodes.sum())
                            + 2 * inst.Hkv * inst.D * int(inst.num_nodes.sum()))
                       + 8 * inst.B * inst.T_max * W)
    return flops, attn_bytes


def accept_bytes(inst, res):
    """Bytes the accept step reads: the logits row of every visited node (the
    root and the accepted nodes) and the draft row of the visited nodes with a
    rejection, counted as min(passes, visited) rows per sequence."""
    sz = 2 if inst.logit_dtype == "bf16" else 4
    visited = res["out_count"].astype(float)
    q_rows = [min(float(p), v) for p, v in zip(res["out_passes"], visited)]
    return float(sz * inst.V * visited.sum() + 4 * inst.V * sum(q_rows))


def time_launches(fn, n, stream):
    """Average duration (ms) of n calls of fn, HIP events on the launch stream."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def attn_build_hash():
    """sha256 of the attention source and the compiler flags it is built with
    (include paths left out, since they name the checkout's location)."""
    from eagle_tree_verification_attn_amd import build as B
    flags = [f for f in B.CFLAGS + B.FILE_FLAGS.get("attn.hip", []) if f != "-I" and os.sep not in f]
    h = hashlib.sha256(open(ATTN_SRC, "rb").read())
    h.update(" ".join(flags).encode())
    return h.hexdigest()


def counters_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it covers this workload (the counters are taken on the
    default one) and was taken on the current kernel source and flags; else
    None."""
    if workload != WORKLOAD or not os.path.exists(COUNTERS):
        return None
    try:
        info = json.load(open(COUNTERS))
        if info.get("attn_build_sha256") != attn_build_hash():
            return None
        return float(info["hbm_bytes_per_launch"])
    except Exception:
        return None


def summarize_counters(fetch_csv, write_csv):
    """Per-launch HBM bytes of the attention kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by the ratio
    of the calibration copy's known size to what the same counter read for it."""
    import csv
    import statistics

    def per_dispatch(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        attn = [v for (d, k), v in vals.items() if ATTN_KERNEL in k]
        copy = [v for (d, k), v in vals.items() if COPY_KERNEL in k]
        if not attn or not copy:
            raise SystemExit(f"{path}: no {ATTN_KERNEL} or {COPY_KERNEL} dispatches with {counter}")
        return statistics.mean(attn), statistics.mean(copy), len(attn), len(copy)

    fa, fc, na, nc = per_dispatch(fetch_csv, "FETCH_SIZE")
    wa, wc, _, _ = per_dispatch(write_csv, "WRITE_SIZE")
    f_factor = (COPY_BYTES / 1024.0) / fc
    w_factor = (COPY_BYTES / 1024.0) / wc
    hbm = 1024.0 * (fa * f_factor + wa * w_factor)
    out = {
        "kernel": f"{ATTN_KERNEL} (sv_tree_attn), workload {WORKLOAD}",
        "attn_build_sha256": attn_build_hash(),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o fetch --output-format csv "
            "-- python3 bench.py --kernels-only",
            "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o write --output-format csv "
            "-- python3 bench.py --kernels-only",
            "python3 bench.py --summarize-counters gpurun_out/pmc_fetch/fetch_counter_collection.csv "
            "gpurun_out/pmc_write/write_counter_collection.csv"],
        "attn_dispatches": na, "copy_dispatches": nc,
        "attn_fetch_kib_per_launch": round(fa, 1), "attn_write_kib_per_launch": round(wa, 1),
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib_per_launch": round(fc, 1), "copy_write_kib_per_launch": round(wc, 1),
        "fetch_scale": round(f_factor, 5), "write_scale": round(w_factor, 5),
        "hbm_bytes_per_launch": round(hbm),
    }
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def tree_shape(inst):
    """Drafted nodes (root excluded) and depth of the sequences' trees: one
    number when every sequence has the same, else one per sequence."""
    nodes, depths = [], []
    for b in range(inst.B):
        n = int(inst.num_nodes[b])
        d = [0] * n
        for i in range(1, n):
            d[i] = d[int(inst.parent[b][i])] + 1
        nodes.append(n - 1)
        depths.append(max(d))
    one = lambda xs: xs[0] if len(set(xs)) == 1 else xs
    return one(nodes), one(depths)


def step_distribution(devs, k, stream):
    """Median, 10th and 90th percentile of k single verification steps (ms),
    each between its own events, cycling over the input sets in ``devs``."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        devs[i % len(devs)].verify_step()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"median_ms": round(float(np.median(t)), 5), "p10_ms": round(float(np.percentile(t, 10)), 5),
            "p90_ms": round(float(np.percentile(t, 90)), 5), "steps": k}


def back_to_back(devs, k, stream):
    """ms per step over k steps launched back to back between two events,
    cycling over the input sets in ``devs``."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(k):
        devs[i % len(devs)].verify_step()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / k


def in_step_times(devs, k, stream):
    """Mean duration (ms) of each kernel of the step in the step's own setting:
    k steps, each issued as its three entry points (mask, attention, accept)
    with HIP events around each call on the launch stream, cycling over the
    input sets in ``devs``."""
    import numpy as np
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(k)]
    torch.cuda.synchronize()
    for i, e in enumerate(evs):
        d = devs[i % len(devs)]
        e[0].record(stream)
        d.mask_build()
        e[1].record(stream)
        d.tree_attn()
        e[2].record(stream)
        d.spec_accept()
        e[3].record(stream)
    torch.cuda.synchronize()
    t = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])
    return {"tree_mask_build": float(t[:, 0].mean()), "tree_attn": float(t[:, 1].mean()),
            "spec_accept": float(t[:, 2].mean())}


def prewarm(devs, seconds):
    """Verification steps back to back for about ``seconds`` of wall time,
    untimed, so that the timed steps run at the clock and power state the GPU
    holds under this load (the first ~50 steps after idle run at another
    clock).  Returns (wall ms, steps)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(50):
            devs[n % len(devs)].verify_step()
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return (time.perf_counter() - t0) * 1e3, n


def time_commit(dev, inst, res, n, stream):
    """sv_commit_accepted on the step's accept results, into destination caches
    of L_max = prefix + T_max; returns (ms per launch, bytes moved)."""
    import torch
    import eagle_tree_verification_attn_amd as sv
    dst_shape = (inst.B, inst.Hkv, int(inst.prefix_len.max()) + inst.T_max, inst.D)
    kd = torch.empty(dst_shape, dtype=dev.k_cache.dtype, device=dev.k_cache.device)
    vd = torch.empty_like(kd)
    plen_out = torch.empty_like(dev.prefix_len)
    args = sv.make_commit_args(dev.k_new, dev.v_new, kd, vd, dev.prefix_len, plen_out)
    status = dev.status.clone()
    fn = lambda: sv.sv_commit_accepted(dev.tree, status, dev.out_nodes, dev.out_count, args, stream)
    for _ in range(3):          # the first launch loads the kernel
        fn()
    ms = time_launches(fn, n, stream)
    s = 2 if inst.dtype == "bf16" else 4
    rows = int(res["out_count"][res["status"] == 0].sum())
    return ms, float(2 * 2 * rows * inst.Hkv * inst.D * s)     # K and V rows, read and written


def stream_rates(stream, n=10):
    """Measured HBM rates on this GPU for context: a read-only stream (torch
    row sums over 1 GiB of float32 in rows of 4096: reads 1 GiB, writes 256 KB;
    the fastest of the torch reductions tried) and a copy (1 GiB in, 1 GiB
    out), each averaged over n launches between HIP events."""
    import torch
    nbytes = 1 << 30
    x = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    rows = x.view(-1, 4096)
    for _ in range(2):
        rows.sum(1)
        y.copy_(x)
    read_ms = time_launches(lambda: rows.sum(1), n, stream)
    copy_ms = time_launches(lambda: y.copy_(x), n, stream)
    del x, y, rows
    torch.cuda.empty_cache()
    return {"read_only_GB_s": round(nbytes / (read_ms * 1e-3) / 1e9, 1),
            "copy_GB_s": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1),
            "note": "row sums over 1 GiB float32, rows of 4096 (read-only stream); 1 GiB device copy (read + write)"}


def time_eagle2(inst, n, stream):
    """One EAGLE-2 tree build for the batch: begin, one expand per step with the
    last one fused with the finish (sv_eagle2_expand_finish); k = 8, 6 steps,
    m = T_max - 1 kept nodes (the batch's tree size), synthetic probability
    rows made on the device.  Returns a dict with the build time, the
    probability bytes it reads and their rate, and the time with a separate
    finish call."""
    import torch
    from eagle_tree_verification_attn_amd.problem import DeviceTreeBuilder
    B, V, k, depth, m = inst.B, inst.V, 8, 6, inst.T_max - 1
    g = torch.Generator(device="cuda").manual_seed(7)
    q = []
    for _ in range(depth):
        z = torch.randn((B, k, V), generator=g, device="cuda", dtype=torch.float32) * 3.0
        q.append(torch.softmax(z, dim=2).contiguous())
        del z
    roots = torch.arange(B, dtype=torch.int32, device="cuda")
    tb = DeviceTreeBuilder(B, V, k, depth, m)
    for _ in range(3):
        tb.run(q, roots, stream)
        tb.run(q, roots, stream, fused_last=True)
    ms_sep = time_launches(lambda: tb.run(q, roots, stream), n, stream)
    ms = time_launches(lambda: tb.run(q, roots, stream, fused_last=True), n, stream)
    ok = int((tb.status == 0).sum().item())
    rows = B * (1 + (depth - 1) * k)          # the root's row, then k rows per later step
    nbytes = float(rows * V * 4)
    del q
    return {"workload": f"eagle2_build_b{B}_k{k}_d{depth}_m{m}", "ms": round(ms, 5),
            "ms_separate_finish": round(ms_sep, 5), "q_bytes": nbytes,
            "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "sequences_ok": ok, "note": "before the step, not part of it"}


def time_draft_head(inst, n_launch, stream):
    """The two-stage draft LM head for one sequence's drafter step: 8 positions,
    hidden 8192 (the 70B shape), rank 256, the batch's vocabulary, tiles of
    256 shuffled rows keeping 2 candidates each; inputs made on the device.
    Returns the time, the algorithmic bytes (B and A once, the candidates'
    rows of W) and, for context, the time a full head would need to read W
    once at peak bandwidth."""
    import torch
    import eagle_tree_verification_attn_amd as sv
    N, d, r, n, tile, k_tile = 8, 8192, 256, inst.V, 256, 2
    g = torch.Generator(device="cuda").manual_seed(13)
    bf = torch.bfloat16
    h = torch.randn((N, d), generator=g, device="cuda").to(bf)
    B = (torch.randn((r, d), generator=g, device="cuda") / d ** 0.5).to(bf)
    A = (torch.randn((n, r), generator=g, device="cuda") / r ** 0.5).to(bf)
    W = (torch.randn((n, d), generator=g, device="cuda") / d ** 0.5).to(bf)
    perm = torch.randperm(n, generator=g, device="cuda").to(torch.int32)
    C = -(-n // tile) * k_tile
    u = torch.empty((N, r), dtype=bf, device="cuda")
    ids = torch.empty((N, C), dtype=torch.int32, device="cuda")
    logits = torch.empty((N, C), dtype=torch.float32, device="cuda")
    args = sv.make_head_args(h, B, A, perm, W, u, ids, logits, tile, k_tile)
    for _ in range(3):
        sv.sv_draft_head(args, stream)
    ms = time_launches(lambda: sv.sv_draft_head(args, stream), n_launch, stream)
    nbytes = float(2 * (r * d + n * r + N * C * d) + 4 * n + 8 * N * C)
    full_ms = 2.0 * n * d / (HBM_PEAK_GBS * 1e9) * 1e3
    del W, A
    return {"workload": f"draft_head_n{N}_d{d}_r{r}_v{n}_tile{tile}_k{k_tile}", "ms": round(ms, 5),
            "bytes": nbytes, "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "full_head_read_roofline_ms": round(full_ms, 5), "note": "drafter side, not part of the step"}


def cpu_baseline(inst, seconds):
    """The oracle on a bounded sample: whole sequences (attention for all heads,
    target softmax and walk), scaled to steps/s of the full batch."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    anc, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    done, t0 = 0, time.perf_counter()
    while done < inst.B:
        b = done
        oracle.tree_attention(inst.q, inst.k_new, inst.v_new, inst.k_cache, inst.v_cache,
                              inst.prefix_len, anc, inst.num_nodes, status, inst.dtype,
                              units=[(b, h) for h in range(inst.Hq)])
        oracle.spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits,
                           inst.logit_dtype, inst.q_probs, inst.temperature, inst.u_accept,
                           inst.u_sample, status, seqs=[b])
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    per_step = dt * inst.B / done
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {inst.B} sequences (all heads' attention, softmax, walk) in "
                      f"{dt:.1f} s, scaled to the batch"}


def all_workloads(steps):
    """One line per workload: the verify step (median of single steps between
    HIP events), attention and accept timed inside steps, attention against
    the bf16 MFMA peak (the fp32 workload against the fp32 vector peak) and
    HBM, and the walk against reading every tree row's logits once at peak."""
    import numpy as np
    import torch
    import eagle_tree_verification_attn_amd as sv
    from eagle_tree_verification_attn_amd.problem import DeviceProblem
    from synth import CONFIGS, make_instance
    sv.lib()
    stream = torch.cuda.current_stream()
    for cfg in CONFIGS:
        inst = make_instance(cfg, 0)
        dev = DeviceProblem(inst, device="cuda:0")
        prewarm((dev,), 1.0)
        step = step_distribution((dev,), steps, stream)
        ins = in_step_times((dev,), steps, stream)
        attn_ms, acc_ms = ins["tree_attn"], ins["spec_accept"]
        res = dev.accept_results()
        flops, attn_bytes = algorithmic_work(inst)
        peak = MFMA_BF16_PEAK_TFLOPS if inst.dtype == "bf16" else 157.3
        sz = 2 if inst.logit_dtype == "bf16" else 4
        every_row_ms = sz * inst.V * float(inst.num_nodes.sum()) / (HBM_PEAK_GBS * 1e9) * 1e3
        print(json.dumps({
            "workload": cfg["name"], "step_median_ms": step["median_ms"],
            "steps_per_s": round(1e3 / step["median_ms"], 1),
            "tree_attn_ms": round(attn_ms, 5), "spec_accept_ms": round(acc_ms, 5),
            "attn_TFLOP_s": round(flops / (attn_ms * 1e-3) / 1e12, 2),
            "attn_frac_of_peak": round(flops / (attn_ms * 1e-3) / 1e12 / peak, 4),
            "attn_peak_TFLOP_s": peak,
            "attn_frac_hbm": round(attn_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "walk_vs_every_row_once": round(acc_ms / every_row_ms, 3),
            "emitted_per_seq": round(float(np.mean(res["out_count"])), 3)}), flush=True)
        del dev, inst
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-seconds", type=float, default=2.0,
                    help="untimed steps for this long before the warm-up steps (clock and power settle)")
    ap.add_argument("--config", default=WORKLOAD)
    ap.add_argument("--kv-shards", type=int, default=1,
                    help="time one GPU's share of the workload when the target is tensor-parallel over "
                         "this many GPUs (attention sharded by KV head: Hq / n and Hkv / n heads)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels-only", action="store_true",
                    help="launch the kernels a few times plus a 1 GiB copy (for rocprofv3)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--all-workloads", action="store_true",
                    help="time the verify step of every workload (one JSON line each), not the headline line")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.all_workloads:
        all_workloads(args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(sequences shard across GPUs with no communication: run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import eagle_tree_verification_attn_amd as sv
    from eagle_tree_verification_attn_amd.problem import DeviceProblem
    from synth import config_by_name, kv_head_shard, make_instance

    sv.lib()   # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    cfg = kv_head_shard(config_by_name(args.config), args.kv_shards)
    t0 = time.perf_counter()
    inst = make_instance(cfg, 0)
    gen_s = time.perf_counter() - t0
    dev = DeviceProblem(inst, device="cuda:0")
    stream = torch.cuda.current_stream()
    print(f"bench: {cfg['name']} generated in {gen_s:.1f} s, uploaded", file=sys.stderr, flush=True)

    if args.kernels_only:
        for _ in range(3):
            dev.verify_step()
        for _ in range(5):
            dev.tree_attn()
        for _ in range(5):
            dev.spec_accept()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)      # calibration: reads and writes COPY_BYTES once
        torch.cuda.synchronize()
        print(f"bench: kernels-only done (copy size {COPY_BYTES} bytes)", file=sys.stderr, flush=True)
        return

    # A second input set of the same shape (seed 1): the timed steps alternate
    # between the two, so every step's inputs were last touched two steps and
    # 2.7 GB of traffic earlier, past the 256 MB Infinity Cache (cold inputs,
    # still resident in HBM).
    inst1 = make_instance(cfg, 1)
    other = DeviceProblem(inst1, device="cuda:0")
    devs = (dev, other)
    pw_ms, pw_steps = prewarm(devs, args.prewarm_seconds)
    print(f"bench: pre-warm {pw_steps} steps in {pw_ms:.0f} ms", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        devs[i % 2].verify_step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        devs[i % 2].verify_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    print(f"bench: {args.steps} steps, {ms_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})",
          file=sys.stderr, flush=True)

    # the distribution of single steps (events around each step, same
    # alternation), each kernel's duration inside steps, then the same input
    # set every step (warm caches)
    per_step = step_distribution(devs, args.steps, stream)
    n = max(200, args.steps)   # ~0.12 s: enough launches for a stable mean
    in_step = in_step_times(devs, n, stream)
    warm_ms = back_to_back((dev,), args.steps, stream)
    res1 = other.accept_results()
    del other, devs
    torch.cuda.empty_cache()

    mask_ms, attn_ms, acc_ms = in_step["tree_mask_build"], in_step["tree_attn"], in_step["spec_accept"]
    # attention launched back to back on its own (no walk between launches:
    # the chip runs it at a lower clock than inside steps), for context
    attn_alone_ms = time_launches(dev.tree_attn, n, stream)
    res = dev.accept_results()
    # the commit of the accepted path (not part of the step): into caches with
    # room after the prefix, so the step's own caches stay as they are
    commit_ms, commit_bytes = time_commit(dev, inst, res, n, stream)
    e2 = time_eagle2(inst, n, stream)
    head = time_draft_head(inst, n, stream)
    rates = stream_rates(stream)
    for d in (e2, head):
        d["frac_of_measured_read"] = round(d["GB_s"] / rates["read_only_GB_s"], 4)
    # the in-step means alternate over the two input sets, so their work is
    # the mean of the two sets' (the same when both sets' trees have one
    # shape, as in the default workload; not with trees of random size)
    w0, w1 = algorithmic_work(inst), algorithmic_work(inst1)
    flops, attn_bytes = (w0[0] + w1[0]) / 2, (w0[1] + w1[1]) / 2

    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    attn_gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
    acc_bytes = (accept_bytes(inst, res) + accept_bytes(inst1, res1)) / 2
    acc_gbs = acc_bytes / (acc_ms * 1e-3) / 1e9
    sz_logit = 2 if inst.logit_dtype == "bf16" else 4
    every_row_bytes = float(sz_logit * inst.V * (int(inst.num_nodes.sum()) + int(inst1.num_nodes.sum())) / 2)
    every_row_ms = every_row_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    traffic = counters_traffic(cfg["name"])
    roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "k_attn_bf16 (sv_tree_attn)",
                "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(attn_ms, 5),
                "launch_timing": "mean of HIP events around each sv_tree_attn call inside steps issued as "
                                 "mask, attention, accept (inputs alternating as in the timed steps)",
                "avg_launch_ms_back_to_back": round(attn_alone_ms, 5)}

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inst, args.cpu_seconds)

    # the trees of both input sets (one entry when they have the same shape)
    shapes = [tree_shape(inst), tree_shape(inst1)]
    tree_nodes = shapes[0][0] if shapes[0] == shapes[1] else [sh[0] for sh in shapes]
    tree_depth = shapes[0][1] if shapes[0] == shapes[1] else [sh[1] for sh in shapes]
    out = {
        "metric": METRIC,
        "value": round(1000.0 / ms_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "B": cfg["B"], "Hq": cfg["Hq"], "Hkv": cfg["Hkv"],
                   "D": cfg["D"], "prefix_len": cfg["prefix_len"], "tree_nodes": tree_nodes,
                   "depth": tree_depth, "V": cfg["V"], "temperature": cfg["tau"],
                   "parallelism": ("single GPU" if args.kv_shards == 1 else
                                   f"one GPU's share of a {args.kv_shards}-way KV-head split (accept not split)")},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels_ms": {"tree_mask_build": round(mask_ms, 5), "tree_attn": round(attn_ms, 5),
                       "spec_accept": round(acc_ms, 5), "note": "inside steps (each entry point between events)"},
        "inputs": "two input sets alternating (no step finds its inputs in the caches)",
        "prewarm": {"ms": round(pw_ms, 1), "steps": pw_steps},
        "per_step": per_step,
        "warm_inputs": {"ms_per_step": round(warm_ms, 5), "steps_per_s": round(1e3 / warm_ms, 2),
                        "note": "one input set every step (caches warm); not the headline"},
        "commit_accepted": {"ms": round(commit_ms, 5), "bytes": commit_bytes,
                            "note": "after the step, not part of it"},
        "eagle2_build": e2,
        "draft_head": head,
        "hbm_roofline": {"tree_attn_verify": {"algorithmic_bytes": attn_bytes,
                                              "GB_s": round(attn_gbs, 1),
                                              "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                                              "frac_of_measured_read": round(attn_gbs / rates["read_only_GB_s"], 4)},
                         "tree_spec_accept": {"algorithmic_bytes": acc_bytes,
                                              "GB_s": round(acc_gbs, 1),
                                              "frac": round(acc_gbs / HBM_PEAK_GBS, 4),
                                              # the same results from a softmax over every tree
                                              # row would read each logits row once: that
                                              # read's time at peak, against this walk's time
                                              "every_row_once_bytes": every_row_bytes,
                                              "every_row_once_roofline_ms": round(every_row_ms, 5),
                                              "walk_ms_vs_that_roofline": round(acc_ms / every_row_ms, 4)},
                         "measured_stream": rates},
        # over both input sets, like the timed steps
        "emitted_tokens_per_seq": round(float(np.mean(np.concatenate([res["out_count"], res1["out_count"]]))), 3),
        "vocab_passes_per_seq": round(float(np.mean(np.concatenate([res["out_passes"], res1["out_passes"]]))), 3),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
