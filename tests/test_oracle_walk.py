"""Pins for the oracle's target softmax, sampler and accept walk (CPU only).

* softmax: a library softmax (scipy), normalisation, shift invariance;
* argmax / inverse CDF: brute force and numpy's searchsorted;
* greedy: brute force over every root-to-leaf path (longest argmax-matching
  prefix, then the argmax at its end);
* chain: the expected number of tokens per target forward
  (1 - alpha^(K+1)) / (1 - alpha), with the worked value the lesson page prints;
* losslessness: total-variation distance between the first emitted token and
  the target distribution < 0.01 over 1e5 walks (chain, i.i.d. siblings,
  without-replacement siblings, a depth-3 tree), and the two-token joint law;
* negative control: the same walk with the sibling proposal update dropped is
  detectably biased;
* residual law: after a rejection, the correction is distributed as
  (p - q)+ normalised;
* input rules: draft tokens in [0, V) (the root's token unread), draft
  probabilities required at temperature > 0 only;
* special cases: q = p always accepts; p(x) = 0 always rejects; one-hot p and
  q reproduce the greedy walk.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
from walk_sim import PathModel, build_tree, run_walk, tv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
WOR, IID = oracle.SIB_WITHOUT_REPLACEMENT, oracle.SIB_IID
TRIALS = 100_000


# ----------------------------------------------------------------------------- softmax / sampler
@pytest.mark.parametrize("tau", [1.0, 0.8, 0.7, 2.5])
def test_target_distribution_matches_library_softmax(tau):
    rng = np.random.default_rng(0)
    z = rng.normal(0, 3, 5000)
    p = oracle.target_distribution(z, tau)
    ref = scipy.special.softmax(z / float(np.float32(tau)))
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)
    assert abs(p.sum() - 1) < 1e-12
    np.testing.assert_allclose(oracle.target_distribution(z + 17.25, tau), p, rtol=1e-10)


def test_argmax_lowest_index_on_ties():
    rng = np.random.default_rng(1)
    for _ in range(200):
        z = rng.integers(0, 6, size=int(rng.integers(1, 40))).astype(np.float64)
        best = 0
        for i in range(z.size):          # brute force: strictly greater moves the winner
            if z[i] > z[best]:
                best = i
        assert oracle.argmax_lowest(z) == best


def test_inverse_cdf_matches_searchsorted_and_margin():
    rng = np.random.default_rng(2)
    for _ in range(500):
        V = int(rng.integers(1, 12))
        P = rng.dirichlet(np.ones(V))
        P[rng.random(V) < 0.3] = 0.0
        if P.sum() == 0:
            P[0] = 1.0
        P /= P.sum()
        u = float(rng.random())
        v, margin = oracle.inverse_cdf(P, u)
        c = np.cumsum(P)
        ref = int(np.searchsorted(c, u, side="right"))
        if ref >= V:
            ref = int(np.nonzero(P > 0)[0][-1])
        assert v == ref and P[v] > 0
        lo = c[v - 1] if v > 0 else None
        want = abs(c[v] - u) if lo is None else min(abs(c[v] - u), abs(u - lo))
        assert margin == pytest.approx(want)
    # hand example: CDF 0.2, 0.5, 1.0
    assert oracle.inverse_cdf(np.array([0.2, 0.3, 0.5]), 0.49)[0] == 1
    assert oracle.inverse_cdf(np.array([0.2, 0.3, 0.5]), 0.5)[0] == 2
    assert oracle.inverse_cdf(np.array([0.2, 0.3, 0.5]), 0.0)[0] == 0


# ----------------------------------------------------------------------------- greedy
def _brute_greedy(parent, tokens, T, Z):
    kids = {i: [] for i in range(T)}
    for i in range(1, T):
        kids[int(parent[i])].append(i)
    best_path = []
    stack = [(0, [])]
    while stack:                      # every root-to-node path that matches argmax all along
        n, path = stack.pop()
        if len(path) > len(best_path):
            best_path = path
        for c in kids[n]:
            if tokens[c] == int(np.argmax(Z[n])):
                stack.append((c, path + [c]))
    end = best_path[-1] if best_path else 0
    return best_path, [int(tokens[c]) for c in best_path] + [int(np.argmax(Z[end]))]


@pytest.mark.parametrize("seed", range(20))
def test_greedy_walk_equals_brute_force(seed):
    from synth import tree_from_widths
    rng = np.random.default_rng(seed)
    V = 6
    parent = tree_from_widths([int(w) for w in rng.integers(1, 4, size=4)], rng)
    T = len(parent)
    Z = rng.normal(size=(T, V))
    Z[rng.random((T, V)) < 0.2] = 5.0           # ties at the maximum
    tokens = np.zeros(T, dtype=np.int64)
    for n in range(T):                            # unique sibling tokens, argmax likely
        kids = [i for i in range(1, T) if parent[i] == n]
        am = int(np.argmax(Z[n]))
        cand = [int(v) for v in rng.permutation(V) if v != am][:len(kids)]
        if kids and rng.random() < 0.7:
            cand[int(rng.integers(len(kids)))] = am
        for j, c in enumerate(rng.permutation(kids)):
            tokens[c] = cand[j]
    for n in range(T):                            # keep siblings unique
        kids = [i for i in range(1, T) if parent[i] == n]
        assert len({int(tokens[c]) for c in kids}) == len(kids)
    w = oracle.accept_walk(parent, tokens, T, lambda n: Z[n], None, 0.0, np.zeros(T),
                           np.zeros(T))
    path, emitted = _brute_greedy(parent, tokens, T, Z)
    assert w["nodes"] == path and w["emitted"] == emitted and w["count"] == len(path) + 1
    assert w["passes"] == 0


# ----------------------------------------------------------------------------- chain length
def test_chain_expected_tokens_closed_form_and_lesson_value():
    g = json.load(open(os.path.join(GOLDEN, "lesson_expected_tokens.json")))
    a, K = g["alpha"], g["K"]
    closed = (1 - a ** (K + 1)) / (1 - a)
    assert round(closed, g["printed_decimals"]) == g["tokens_per_forward_printed"]
    # simulate: identical (p, q) at every position with sum(min(p, q)) = alpha
    p, q = np.array([0.9, 0.1]), np.array([0.7, 0.3])
    assert np.minimum(p, q).sum() == pytest.approx(a)
    model = PathModel(2, 0, fixed=(p, q))
    rng = np.random.default_rng(11)
    counts = []
    for _ in range(TRIALS):
        par, tok, ctx = build_tree(model, (), [1] * K, "iid", rng)
        counts.append(run_walk(oracle, model, par, tok, ctx, rng, WOR)["count"])
    assert abs(np.mean(counts) - closed) < 0.02


@pytest.mark.parametrize("K", [1, 2, 6])
def test_chain_expected_tokens_other_lengths(K):
    p, q = np.array([0.5, 0.3, 0.2]), np.array([0.2, 0.3, 0.5])
    a = np.minimum(p, q).sum()
    closed = (1 - a ** (K + 1)) / (1 - a)
    model = PathModel(3, 0, fixed=(p, q))
    rng = np.random.default_rng(12 + K)
    n = 40_000
    c = [run_walk(oracle, model, *build_tree(model, (), [1] * K, "iid", rng), rng, WOR)["count"]
         for _ in range(n)]
    assert abs(np.mean(c) - closed) < 4 * np.std(c) / np.sqrt(n)


# ----------------------------------------------------------------------------- losslessness
def _first_token_tv(model, widths, mode, walk_mode, seed, trials=TRIALS):
    rng = np.random.default_rng(seed)
    counts = np.zeros(model.V)
    for _ in range(trials):
        par, tok, ctx = build_tree(model, (), widths, mode, rng)
        w = run_walk(oracle, model, par, tok, ctx, rng, walk_mode)
        counts[w["emitted"][0]] += 1
    return tv(counts, model.pq(())[0])


@pytest.mark.parametrize("seed,widths,mode,walk_mode", [
    (101, [1, 1, 1], "iid", WOR),          # chain
    (102, [3], "iid", IID),                # i.i.d. siblings, k = 3
    (103, [3], "wor", WOR),                # siblings without replacement, k = 3
    (104, [2, 2, 1], "wor", WOR),          # depth-3 tree
])
def test_first_token_total_variation(seed, widths, mode, walk_mode):
    model = PathModel(8, 5, conc_p=1.0, conc_q=1.0)
    assert _first_token_tv(model, widths, mode, walk_mode, seed=seed) < 0.01


NEG_P = np.array([0.106, 0.031, 0.533, 0.036, 0.011, 0.178, 0.049, 0.056])
NEG_Q = np.array([0.006, 0.157, 0.214, 0.047, 0.345, 0.043, 0.162, 0.026])


def test_sibling_rule_with_and_without_proposal_update():
    """Siblings drawn without replacement: with the proposal update the law is
    exact; walking them as if i.i.d. (update dropped) is biased (TV ~ 0.06)."""
    model = PathModel(8, 0, fixed=(NEG_P, NEG_Q))
    good = _first_token_tv(model, [3], "wor", WOR, seed=21)
    bad = _first_token_tv(model, [3], "wor", IID, seed=21)
    assert good < 0.01
    assert bad > 0.03


def test_two_token_joint_law():
    """Joint law of the first two emitted tokens equals p(x1) p(x2 | x1)."""
    V = 4
    model = PathModel(V, 9)
    rng = np.random.default_rng(31)
    counts = np.zeros((V, V))
    for _ in range(TRIALS):
        par, tok, ctx = build_tree(model, (), [2, 2], "wor", rng)
        w = run_walk(oracle, model, par, tok, ctx, rng, WOR)
        e = w["emitted"]
        if len(e) >= 2:
            counts[e[0], e[1]] += 1
        else:                       # one token emitted: verify the next step from it
            par2, tok2, ctx2 = build_tree(model, (e[0],), [2, 2], "wor", rng)
            w2 = run_walk(oracle, model, par2, tok2, ctx2, rng, WOR)
            counts[e[0], w2["emitted"][0]] += 1
    p1 = model.pq(())[0]
    joint = np.array([[p1[a] * model.pq((a,))[0][b] for b in range(V)] for a in range(V)])
    assert tv(counts.ravel(), joint.ravel()) < 0.01


def test_residual_law_after_rejection():
    p, q = np.array([0.5, 0.1, 0.3, 0.1]), np.array([0.1, 0.6, 0.1, 0.2])
    model = PathModel(4, 0, fixed=(p, q))
    rng = np.random.default_rng(41)
    counts = np.zeros(4)
    for _ in range(TRIALS):
        par, tok, ctx = build_tree(model, (), [1], "iid", rng)
        w = run_walk(oracle, model, par, tok, ctx, rng, WOR)
        if not w["nodes"]:
            counts[w["emitted"][0]] += 1
    r = np.maximum(p - q, 0)
    assert tv(counts, r / r.sum()) < 0.01


def test_temperature_scales_logits():
    rng = np.random.default_rng(51)
    z = rng.normal(0, 1.5, 6)
    tau = 0.7
    P = scipy.special.softmax(z / float(np.float32(tau)))
    counts = np.zeros(6)
    for _ in range(50_000):       # root-only tree: the emitted token is the bonus draw
        w = oracle.accept_walk(np.array([-1]), np.array([0]), 1, lambda n: z, None, tau,
                               rng.random(1), rng.random(1))
        counts[w["emitted"][0]] += 1
    assert tv(counts, P) < 0.01


# ----------------------------------------------------------------------------- special cases
def test_q_equal_p_accepts_first_children():
    rng = np.random.default_rng(61)
    from synth import tree_from_widths
    for _ in range(50):
        parent = tree_from_widths([3, 2, 2], rng)
        T = len(parent)
        Z = rng.normal(size=(T, 10))
        Qs = np.array([scipy.special.softmax(Z[n]) for n in range(T)])
        tokens = rng.integers(0, 10, size=T)
        w = oracle.accept_walk(parent, tokens, T, lambda n: Z[n], lambda n: Qs[n], 1.0,
                               rng.random(T), rng.random(T), IID)
        n, chain = 0, []
        while True:
            kids = [i for i in range(1, T) if parent[i] == n]
            if not kids:
                break
            chain.append(kids[0])
            n = kids[0]
        assert w["nodes"] == chain and w["count"] == len(chain) + 1


def test_zero_target_probability_always_rejects():
    z = np.array([0.0, -np.inf, 1.0, 0.5])
    q = np.array([0.25, 0.25, 0.25, 0.25])
    rng = np.random.default_rng(71)
    for _ in range(200):
        w = oracle.accept_walk(np.array([-1, 0]), np.array([0, 1]), 2, lambda n: z,
                               lambda n: q, 1.0, rng.random(2), rng.random(2))
        assert w["nodes"] == [] and w["emitted"][0] != 1


def test_one_hot_p_and_q_reduce_to_greedy():
    rng = np.random.default_rng(81)
    from synth import tree_from_widths
    V = 5
    for _ in range(50):
        parent = tree_from_widths([2, 2, 2], rng)
        T = len(parent)
        hot = rng.integers(0, V, size=T)
        Z = np.full((T, V), -np.inf)
        Z[np.arange(T), hot] = 0.0
        Zg = np.where(np.isfinite(Z), 1.0, 0.0)
        tokens = rng.integers(0, V, size=T)
        for i in range(1, T):
            if rng.random() < 0.6:
                tokens[i] = hot[parent[i]]
        # each draft row q is one-hot on the first child's token (the drafter's choice)
        Q = np.zeros((T, V))
        for n in range(T):
            kids = [i for i in range(1, T) if parent[i] == n]
            Q[n, tokens[kids[0]] if kids else 0] = 1.0
        sto = oracle.accept_walk(parent, tokens, T, lambda n: Z[n], lambda n: Q[n], 1.0,
                                 rng.random(T), rng.random(T), IID)
        gre = oracle.accept_walk(parent, tokens, T, lambda n: Zg[n], None, 0.0, np.zeros(T),
                                 np.zeros(T))
        assert sto["nodes"] == gre["nodes"] and sto["emitted"] == gre["emitted"]


# ----------------------------------------------------------------------------- input rule
def _two_child_tree_instance(V=12):
    """Root with children 1, 2; node 1 has child 3.  q = p at every node, so the
    walk accepts the first child at each node (special case above) and visits
    rows 0, 1 and 3, never row 2."""
    rng = np.random.default_rng(5)
    parent = np.array([[-1, 0, 0, 1]], dtype=np.int32)
    z = rng.normal(size=(1, 4, V)).astype(np.float32)
    q = scipy.special.softmax(z.astype(np.float64), axis=-1).astype(np.float32)
    tokens = np.array([[0, 3, 4, 5]], dtype=np.int32)
    return parent, z, q, tokens, rng.random((1, 4)).astype(np.float32), rng.random((1, 4)).astype(np.float32)


@pytest.mark.parametrize("row,bad", [(2, np.nan), (2, np.inf), (0, np.nan), (1, -np.inf), (3, np.inf)])
def test_nonfinite_logits_only_in_rows_the_walk_reads(row, bad):
    parent, z, q, tokens, ua, us = _two_child_tree_instance()
    num = np.array([4], dtype=np.int32)
    clean = oracle.spec_accept(parent, num, tokens, z, "f32", q, np.ones(1, np.float32), ua, us,
                               np.zeros(1, np.int32), IID)
    assert clean["out_nodes"][0, :2].tolist() == [1, 3]      # q = p: first children accepted
    z2 = z.copy()
    z2[0, row, 7] = bad
    res = oracle.spec_accept(parent, num, tokens, z2, "f32", q, np.ones(1, np.float32), ua, us,
                             np.zeros(1, np.int32), IID)
    if row == 2:   # never visited: the outcome is unchanged
        assert res["status"][0] == oracle.TREE_OK
        np.testing.assert_array_equal(res["out_tokens"], clean["out_tokens"])
    else:
        assert res["status"][0] == oracle.TREE_E_NONFINITE
        assert res["out_count"][0] == 0 and (res["out_nodes"] == -1).all()


def _spec_accept_one(parent, tokens, z, q, tau, ua, us):
    num = np.array([parent.shape[1]], dtype=np.int32)
    return oracle.spec_accept(parent, num, tokens, z, "f32", q, np.array([tau], np.float32), ua, us,
                              np.zeros(1, np.int32), IID)


@pytest.mark.parametrize("pos,value,want", [
    (1, 12, oracle.TREE_E_TOKEN),    # = V: one past the last vocabulary id
    (3, 12, oracle.TREE_E_TOKEN),    # a deeper node
    (2, -1, oracle.TREE_E_TOKEN),    # negative, on a node the walk never visits
    (1, 11, oracle.TREE_OK),         # V - 1: the last valid id
    (1, 0, oracle.TREE_OK),          # the first valid id
    (0, -7, oracle.TREE_OK),         # the root's token: never a candidate, not read
    (0, 12, oracle.TREE_OK),
])
def test_token_range_rule(pos, value, want):
    """A draft token indexes the vocabulary rows p and q (the lesson's
    "Exactness rule" reads p(x) and q(x)), so every draft token must lie in
    [0, V); one outside makes the sequence invalid with count 0 and -1
    outputs, wherever the node sits in the tree.  The root is the last
    emitted token, not a candidate, so its token is not checked."""
    parent, z, q, tokens, ua, us = _two_child_tree_instance(V=12)
    tokens = tokens.copy()
    tokens[0, pos] = value
    res = _spec_accept_one(parent, tokens, z, q, 1.0, ua, us)
    assert res["status"][0] == want
    if want == oracle.TREE_OK:
        if pos == 0:   # the outcome does not depend on the root's token
            clean = _spec_accept_one(parent, _two_child_tree_instance(V=12)[3], z, q, 1.0, ua, us)
            np.testing.assert_array_equal(res["out_tokens"], clean["out_tokens"])
        assert res["out_count"][0] >= 1
    else:
        assert res["out_count"][0] == 0 and (res["out_nodes"] == -1).all() and (res["out_tokens"] == -1).all()
        assert res["walks"][0] is None


@pytest.mark.parametrize("tau,want", [(1.0, oracle.TREE_E_NOQ), (0.25, oracle.TREE_E_NOQ),
                                      (0.0, oracle.TREE_OK), (-1.0, oracle.TREE_OK)])
def test_missing_q_rule(tau, want):
    """Stochastic verification divides by q(x) (the lesson's "Exactness
    rule"), so a sequence at temperature > 0 without draft probabilities is
    invalid; greedy verification compares with argmax p only and needs no q,
    and then gives the same result as with q present."""
    parent, z, q, tokens, ua, us = _two_child_tree_instance(V=12)
    res = _spec_accept_one(parent, tokens, z, None, tau, ua, us)
    assert res["status"][0] == want
    if want == oracle.TREE_E_NOQ:
        assert res["out_count"][0] == 0 and (res["out_nodes"] == -1).all() and (res["out_tokens"] == -1).all()
    else:
        with_q = _spec_accept_one(parent, tokens, z, q, tau, ua, us)
        np.testing.assert_array_equal(res["out_tokens"], with_q["out_tokens"])
        np.testing.assert_array_equal(res["out_nodes"], with_q["out_nodes"])
        # the emitted token is the argmax of the last visited node's row
        last = 0 if res["out_count"][0] == 1 else int(res["out_nodes"][0, res["out_count"][0] - 2])
        assert res["out_tokens"][0, res["out_count"][0] - 1] == int(np.argmax(z[0, last]))


def test_missing_q_rule_per_sequence():
    """The rule is per sequence: in a batch with mixed temperatures and no q,
    only the stochastic sequences are invalid."""
    parent, z, q, tokens, ua, us = _two_child_tree_instance(V=12)
    B = 4
    P = np.repeat(parent, B, 0)
    res = oracle.spec_accept(P, np.full(B, 4, np.int32), np.repeat(tokens, B, 0), np.repeat(z, B, 0), "f32", None,
                             np.array([0.0, 1.0, 0.0, 0.7], np.float32), np.repeat(ua, B, 0),
                             np.repeat(us, B, 0), np.zeros(B, np.int32), IID)
    assert res["status"].tolist() == [oracle.TREE_OK, oracle.TREE_E_NOQ, oracle.TREE_OK, oracle.TREE_E_NOQ]
    assert res["out_count"].tolist()[1::2] == [0, 0]
