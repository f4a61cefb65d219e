"""Pins for the oracle's EAGLE-2 tree builder (CPU only).

* a hand-worked example in the setting of the article's Figures 2-5 and 2-6
  (k = 2), including the tie between a shallow and a deep node of equal value;
* brute force: the kept set is connected and has the largest total value of
  all connected subtrees of m draft nodes;
* path products: every kept node's value equals the product of the input
  probabilities along its path, read back through the output's parent and
  q-row arrays;
* the layer selection: every frontier node is worth at least every node of
  its layer that was not selected;
* closed forms: node counts per depth, and the chain (k = 1) following the
  most probable token of each row;
* invalid rows: a probability outside [0, 1] or a NaN marks the sequence.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import eagle2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "eagle2_expand_rerank_example.json")) as f:
        return json.load(f)


def _golden_q(g):
    k = g["k"]
    q0 = np.zeros((k, g["V"]), dtype=np.float32)
    q0[0] = g["q_step0_row0"]
    q1 = np.asarray(g["q_step1_rows"], dtype=np.float32)
    return [q0, q1]


@pytest.mark.parametrize("m", [2, 3, 4, 6])
def test_hand_worked_example(m):
    g = _golden()
    r = eagle2.build_sequence(_golden_q(g), g["root_token"], g["k"], g["depth"], m)
    assert r["status"] == eagle2.TREE_OK
    vals = [float(n["value"]) for n in r["nodes"]]
    np.testing.assert_allclose(vals, g["values_by_creation"], rtol=1e-6)
    assert [n["token"] for n in r["nodes"]] == g["tokens_by_creation"]
    assert [n["parent"] for n in r["nodes"]] == g["parents_by_creation"]
    exp = g["expected"][f"m{m}"]
    assert r["parent"].tolist() == exp["parent"]
    assert r["tokens"].tolist() == exp["tokens"]
    assert r["q_row"].tolist() == exp["q_row"]
    assert r["frontiers"] == [[0], [1, 2]]


def _random_q(rng, k, depth, V, sharp=2.0):
    out = []
    for s in range(depth):
        z = rng.normal(0, sharp, (k, V))
        p = np.exp(z - z.max(axis=1, keepdims=True))
        out.append((p / p.sum(axis=1, keepdims=True)).astype(np.float32))
    return out


def _subtree_sets(nodes, m):
    """All connected (ancestor-closed) sets of m draft nodes, by brute force."""
    draft = [n["id"] for n in nodes if n["id"] != 0]
    par = {n["id"]: n["parent"] for n in nodes}
    for comb in itertools.combinations(draft, m):
        s = set(comb)
        if all(par[i] == 0 or par[i] in s for i in s):
            yield s


@pytest.mark.parametrize("seed,k,depth,m", [(0, 2, 2, 3), (1, 2, 3, 4), (2, 3, 2, 5), (3, 2, 3, 6),
                                            (4, 3, 3, 4), (5, 2, 2, 6)])
def test_kept_set_is_the_best_connected_subtree(seed, k, depth, m):
    rng = np.random.default_rng(seed)
    q = _random_q(rng, k, depth, 12)
    r = eagle2.build_sequence(q, 3, k, depth, m)
    kept = set(r["order"][1:])
    val = {n["id"]: float(n["value"]) for n in r["nodes"]}
    best = max(sum(val[i] for i in s) for s in _subtree_sets(r["nodes"], m))
    assert abs(sum(val[i] for i in kept) - best) <= 1e-6 * max(1.0, best)
    par = {n["id"]: n["parent"] for n in r["nodes"]}
    assert all(par[i] == 0 or par[i] in kept for i in kept)


@pytest.mark.parametrize("seed", range(5))
def test_values_are_path_products_of_the_input_rows(seed):
    rng = np.random.default_rng(100 + seed)
    k, depth, m, V = 4, 4, 20, 50
    q = _random_q(rng, k, depth, V)
    r = eagle2.build_sequence(q, 7, k, depth, m)
    parent, tokens, q_row = r["parent"], r["tokens"], r["q_row"]
    T = len(parent)
    assert T == m + 1 and parent[0] == -1
    for i in range(1, T):
        assert parent[i] < i
        # product over the path, each edge's probability read from the row
        # that expanded the edge's parent
        prod = np.float32(1.0)
        j = i
        path = []
        while j > 0:
            path.append(j)
            j = parent[j]
        for j in reversed(path):
            row = q_row[parent[j]]
            assert row >= 0
            prod = np.float32(prod * q[row // k][row % k][tokens[j]])
        node = r["nodes"][r["order"][i]]
        assert prod == node["value"]


@pytest.mark.parametrize("seed", range(4))
def test_frontier_holds_the_best_of_each_layer(seed):
    rng = np.random.default_rng(200 + seed)
    k, depth = 3, 4
    q = _random_q(rng, k, depth, 30)
    r = eagle2.build_sequence(q, 0, k, depth, 10)
    nodes = r["nodes"]
    for s in range(1, depth):
        layer = [n for n in nodes if n["depth"] == s]
        front = set(r["frontiers"][s])
        assert len(front) == min(k, len(layer))
        worst_in = min(float(nodes[i]["value"]) for i in front)
        best_out = max([float(n["value"]) for n in layer if n["id"] not in front], default=-1.0)
        assert worst_in >= best_out


@pytest.mark.parametrize("k,depth", [(2, 3), (3, 2), (4, 3)])
def test_node_counts_closed_form(k, depth):
    rng = np.random.default_rng(k * 10 + depth)
    q = _random_q(rng, k, depth, 40)
    n_gen = eagle2.generated_nodes(k, depth)
    r = eagle2.build_sequence(q, 1, k, depth, n_gen)
    per_depth = np.bincount([n["depth"] for n in r["nodes"]])
    assert per_depth.tolist() == [1, k] + [k * k] * (depth - 1)
    assert len(r["parent"]) == n_gen + 1


def test_chain_when_k_is_one():
    rng = np.random.default_rng(9)
    depth, V = 5, 25
    q = _random_q(rng, 1, depth, V)
    r = eagle2.build_sequence(q, 4, 1, depth, depth)
    assert r["parent"].tolist() == [-1] + list(range(depth))
    assert r["tokens"][1:].tolist() == [int(np.argmax(q[s][0])) for s in range(depth)]


def test_sibling_order_is_descending_probability_and_ties_go_to_lower_token():
    V = 8
    q0 = np.zeros((3, V), dtype=np.float32)
    q0[0] = [0.1, 0.2, 0.0, 0.2, 0.4, 0.0, 0.1, 0.0]
    q = [q0]
    r = eagle2.build_sequence(q, 0, 3, 1, 3)
    assert r["tokens"].tolist() == [0, 4, 1, 3]


@pytest.mark.parametrize("bad", [np.nan, -0.1, 1.5, np.inf])
def test_invalid_probability_marks_the_sequence(bad):
    rng = np.random.default_rng(3)
    q = _random_q(rng, 2, 2, 10)
    q[1][1, 4] = bad
    r = eagle2.build_sequence(q, 0, 2, 2, 3)
    assert r["status"] == eagle2.TREE_E_PROB and r["parent"] is None
    qa = [np.stack([q[s]] * 2) for s in range(2)]
    out = eagle2.build(qa, [0, 0], 2, 2, 3)
    assert out["status"].tolist() == [eagle2.TREE_E_PROB] * 2
    assert out["num_nodes"].tolist() == [0, 0] and (out["parent"] == -1).all()


def test_unread_rows_are_not_checked():
    rng = np.random.default_rng(4)
    q = _random_q(rng, 2, 2, 10)
    q[0][1, 2] = np.nan          # step 0 reads only the root's row
    r = eagle2.build_sequence(q, 0, 2, 2, 3)
    assert r["status"] == eagle2.TREE_OK
