"""GPU EAGLE-2 tree builder (sv_eagle2_*) against the oracle.

Every output is an integer decided by exact float32 comparisons (values are
one IEEE multiply per node on both sides), so parent arrays, tokens, q rows,
frontiers, node counts and statuses must match the oracle bit for bit.
Cases: widths k = 1 .. 16, one to five steps, m from 1 to every generated
node, vocabularies that do and do not split into several chunks and are not
multiples of 4, rows with many equal probabilities (ties), invalid rows read
and not read, and the 32-sequence workload (k = 8, 6 steps, m = 64,
V = 128256) on sampled sequences.  The built trees then run through the
verification kernels.
"""
import numpy as np
import pytest

from oracle import eagle2
from gpu_util import need_gpu, say
from synth import make_draft_rows

pytestmark = pytest.mark.gpu


def _run(B, V, k, depth, m, q_host, roots, fused=False):
    import torch
    from eagle_tree_verification_attn_amd.problem import DeviceTreeBuilder
    dev = DeviceTreeBuilder(B, V, k, depth, m)
    q_dev = [torch.from_numpy(np.ascontiguousarray(q)).cuda() for q in q_host]
    roots_dev = torch.from_numpy(np.asarray(roots, dtype=np.int32)).cuda()
    dev.run(q_dev, roots_dev, fused_last=fused)
    torch.cuda.synchronize()
    return dev.results()


def _check(res, ref, seqs=None, label=""):
    B = res["status"].shape[0]
    for b in (range(B) if seqs is None else seqs):
        assert res["status"][b] == ref["status"][b], (label, b)
        assert res["num_nodes"][b] == ref["num_nodes"][b], (label, b)
        for f in ("parent", "tokens", "q_row"):
            np.testing.assert_array_equal(res[f][b], ref[f][b], err_msg=f"{label} b={b} {f}")
        if ref["status"][b] == eagle2.TREE_OK:
            # frontier of step s + 1 is what expand(s) returns
            D = res["frontier"].shape[0]
            for s in range(D - 1):
                np.testing.assert_array_equal(res["frontier"][s, b], ref["frontier"][s + 1, b],
                                              err_msg=f"{label} b={b} frontier step {s}")


CASES = [
    # B, V, k, depth, m, tie_step
    (3, 500, 2, 2, 4, None),
    (4, 1001, 3, 3, 12, None),          # V not a multiple of 4
    (5, 20000, 4, 3, 20, None),         # several vocabulary chunks
    (2, 3000, 1, 5, 5, None),           # a chain
    (3, 700, 5, 2, 30, None),           # every generated node (5 + 25)
    (2, 400, 16, 2, 200, None),         # widest expansion
    (4, 2000, 8, 4, 1, None),           # keep one node
    (4, 3000, 6, 3, 50, 2.0 ** -10),    # many equal probabilities
    (3, 9000, 4, 4, 30, 2.0 ** -8),     # ties across chunks
]


@pytest.mark.parametrize("fused", [False, True], ids=["finish", "fused_last"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_V{c[1]}_k{c[2]}_d{c[3]}_m{c[4]}{'_ties' if c[5] else ''}" for c in CASES])
def test_builder_matches_oracle(case, fused):
    """fused: the last step runs as sv_eagle2_expand_finish (expand and finish
    in one launch); every output must be the same."""
    need_gpu()
    B, V, k, depth, m, tie = case
    q = make_draft_rows(B, k, depth, V, seed=sum(case[:5]), tie_step=tie)
    roots = np.arange(B, dtype=np.int32) % V
    say(f"eagle2 B={B} V={V} k={k} depth={depth} m={m} ties={tie} fused={fused}")
    ref = eagle2.build(q, roots, k, depth, m)
    res = _run(B, V, k, depth, m, q, roots, fused)
    _check(res, ref, label=str(case))
    # the frontier tokens are the frontier nodes' tokens (the fused last step
    # writes no frontier)
    steps = depth - 1 if fused else depth
    fr, ft = res["frontier"][:steps], res["frontier_tokens"][:steps]
    assert (ft[fr < 0] == -1).all()


@pytest.mark.parametrize("V", [20000, 9001])
def test_builder_heavy_ties(V):
    """Rows where thousands of tokens tie at the k-th value: more keys sit at
    the chunk's bound than its candidate list holds, so the chunk's k best
    come from rounds of a block maximum instead (the path that reads the chunk
    again).  Sequence 0: uniform rows.  Sequence 1: three large values, every
    other token equal.  Sequence 2: ordinary rows.  V = 9001 also covers rows
    that are not 16-byte runs."""
    need_gpu()
    B, k, depth, m = 3, 5, 3, 20
    q = make_draft_rows(B, k, depth, V, seed=V)
    for s in range(depth):
        q[s][0] = np.float32(1.0 / V)
        q[s][1] = np.float32(0.25 / V)
        for j in range(k):
            q[s][1, j, [17 + j, V // 2 + 3 * j, V - 1 - j]] = np.float32([0.3, 0.2, 0.1])
    roots = np.array([1, 2, 3], dtype=np.int32)
    say(f"eagle2 heavy ties V={V}")
    ref = eagle2.build(q, roots, k, depth, m)
    assert (ref["status"] == eagle2.TREE_OK).all()
    res = _run(B, V, k, depth, m, q, roots)
    _check(res, ref, label=f"ties V={V}")
    # uniform rows: the children of every node are the k lowest token ids
    kids = res["tokens"][0][res["parent"][0] == 0]
    assert sorted(kids.tolist()) == list(range(k))


@pytest.mark.parametrize("fused", [False, True], ids=["finish", "fused_last"])
def test_invalid_rows_mark_only_their_sequence(fused):
    need_gpu()
    B, V, k, depth, m = 6, 800, 3, 3, 10
    q = make_draft_rows(B, k, depth, V, seed=77)
    q[1][1, 2, 17] = np.nan          # read (frontier row 2 of step 1)
    q[2][2, 0, 5] = 1.5              # read
    q[1][3, 0, 9] = -0.25            # read
    q[0][4, 1, 3] = np.nan           # not read: step 0 reads only the root's row
    q[0][5, 0, 799] = np.inf         # read, last token
    roots = np.full(B, 3, dtype=np.int32)
    say("eagle2 invalid rows")
    ref = eagle2.build(q, roots, k, depth, m)
    assert ref["status"].tolist() == [0, 10, 10, 10, 0, 10]
    res = _run(B, V, k, depth, m, q, roots, fused)
    _check(res, ref, label="invalid")
    assert (res["parent"][1] == -1).all() and res["num_nodes"][1] == 0


def test_builder_full_workload_sampled():
    need_gpu()
    import torch
    B, V, k, depth, m = 32, 128256, 8, 6, 64
    q = make_draft_rows(B, k, depth, V, seed=4)
    roots = (np.arange(B, dtype=np.int32) * 7919) % V
    say(f"eagle2 full workload B={B} V={V} k={k} depth={depth} m={m}")
    res = _run(B, V, k, depth, m, q, roots)
    fused = _run(B, V, k, depth, m, q, roots, fused=True)
    for f in ("parent", "tokens", "q_row", "num_nodes", "status"):
        np.testing.assert_array_equal(fused[f], res[f], err_msg=f"fused last step: {f}")
    seqs = [0, 5, 13, 31]
    for b in seqs:
        r = eagle2.build_sequence([q[s][b] for s in range(depth)], int(roots[b]), k, depth, m)
        assert res["status"][b] == r["status"] and res["num_nodes"][b] == m + 1
        np.testing.assert_array_equal(res["parent"][b], r["parent"])
        np.testing.assert_array_equal(res["tokens"][b], r["tokens"])
        np.testing.assert_array_equal(res["q_row"][b], r["q_row"])
    # every sequence: a valid tree (parents precede children), m + 1 positions
    assert (res["status"] == 0).all()
    P = res["parent"]
    assert (P[:, 0] == -1).all() and all((P[b, 1:] < np.arange(1, m + 1)).all() and (P[b, 1:] >= 0).all()
                                         for b in range(B))
    del q
    torch.cuda.empty_cache()


def test_built_trees_run_through_verification():
    """Builder output -> mask build, attention and accept, checked against the
    oracle's verification on the same trees (q rows gathered through q_row)."""
    need_gpu()
    import torch
    import oracle
    from gpu_util import sv_problem, check_mask
    from synth import make_instance
    B, V, k, depth, m = 4, 600, 3, 3, 12
    q = make_draft_rows(B, k, depth, V, seed=11)
    roots = np.array([1, 2, 3, 4], dtype=np.int32)
    res = _run(B, V, k, depth, m, q, roots)
    assert (res["status"] == 0).all()
    T = m + 1
    spec = dict(cfg_id=901, B=B, Hq=8, Hkv=2, D=64, dtype="bf16", logit_dtype="bf16", prefix_len=[30, 0, 65, 7],
                tree=("widths", [T - 1]), V=V, tau=[0.0, 0.8, 1.0, 0.7], sigma=1.0, draft_std=3.0,
                sibling_mode="wor")
    inst = make_instance(spec, 0)
    # the built trees and their draft rows replace the synthetic ones
    inst.parent = res["parent"].astype(np.int32)
    inst.tokens = res["tokens"].astype(np.int32)
    inst.num_nodes = res["num_nodes"].astype(np.int32)
    qp = np.zeros((B, T, V), dtype=np.float32)
    for b in range(B):
        for i in range(T):
            r = res["q_row"][b, i]
            if r >= 0:
                qp[b, i] = q[r // k][b, r % k]
    inst.q_probs = qp
    say("eagle2 trees through verification")
    dev = sv_problem(inst)
    dev.verify_step()
    check_mask(dev, inst)
    ref = oracle.verify_step(inst)
    got = dev.attn_result()
    err = np.abs(got - ref["attn"])
    assert (err <= 2e-2 + 1e-2 * np.abs(ref["attn"])).all(), float(err.max())
    acc = dev.accept_results()
    assert (acc["status"] == ref["accept"]["status"]).all()
    for b in range(B):
        w = ref["accept"]["walks"][b]
        if w is not None and w["exempt_at"] is None:
            np.testing.assert_array_equal(acc["out_nodes"][b], ref["accept"]["out_nodes"][b])
            np.testing.assert_array_equal(acc["out_tokens"][b], ref["accept"]["out_tokens"][b])
