"""CPU oracle for the EAGLE-2 draft-tree builder (test infrastructure only).

Like ``oracle.ref`` this is the plain definition of what the GPU builder
computes, used only by the tests (and nothing on the product path).  It shares
no code with the HIP library.

Source: [EAGLE article] (the course.zhidx.com mirror of the Zhihu article on
EAGLE / EAGLE-2 / EAGLE-3 / DFlash), section 2.3 "Context-aware draft tree":

* a node's value is the product of the draft confidences along its path from
  the root, standing in for the probability that the whole path is accepted
  (sec. 2.2 and the "Expansion Phase" paragraph; the formula itself is lost in
  the extracted text);
* expansion: in the newest layer, the top-k nodes by value are fed to the
  draft model and the tokens it proposes are attached as their children
  (Figure 2-5, picture lost);
* reranking: over all draft nodes the top-m by value are kept; a child's
  value never exceeds its parent's and equal values go to the shallower node,
  so the kept set is a connected tree (Figure 2-6, picture lost);
* the kept tree is flattened for verification (section "Flatten + Attention
  mask").

Readings where the page is silent (each is listed in the design notes):

* the draft confidences are the draft model's probabilities, given as input
  rows q (float32, one row of V per expanded node), as they are for
  verification; every expanded node gets as children its k most probable
  tokens (probability descending, ties to the lower token id);
* the root (the last emitted token) has value 1, is expanded at step 0 and is
  position 0 of the output;
* values are float32 products (one IEEE multiply per node), and every
  selection compares them exactly: top-k of a layer by (value descending,
  creation order), rerank by (value descending, depth ascending, creation
  order);
* the flattened order is by depth, then parent position, then the child's
  rank among its siblings (descending probability), so parents precede
  children and siblings appear in the order they were proposed;
* a row that is read and holds a value outside [0, 1] or not a number marks
  the sequence invalid (TREE_E_PROB): no nodes are output.

Pinned by ``tests/test_oracle_eagle2.py``: a hand-worked example in the page's
setting, brute force over all connected subtrees of size m (the kept set must
have the largest total value), path products recomputed from the input rows,
closed-form node counts, the chain special case (k = 1), and the layer
selection checked against every unselected node.
"""
import numpy as np

TREE_OK = 0
TREE_E_PROB = 10


def _top_tokens(row, k):
    """k largest entries of a float32 row: probability descending, then token
    ascending.  Returns (tokens, probabilities)."""
    V = row.shape[0]
    order = np.lexsort((np.arange(V), -row.astype(np.float32)))
    toks = order[:k]
    return toks.astype(np.int64), row[toks].astype(np.float32)


def _row_ok(row):
    r = np.asarray(row, dtype=np.float32)
    return bool(np.all(np.isfinite(r)) and np.all(r >= 0.0) and np.all(r <= 1.0))


def build_sequence(q_steps, root_token, k, depth, m):
    """Build one sequence's tree.

    q_steps[s] is a float32 array [k][V]: the draft probabilities of the rows
    of step s in frontier order (only row 0, the root's, is read at step 0).
    Returns a dict with the generated nodes and the flattened output:
      nodes: list of dicts (id, parent, token, value, depth, rank, q_row)
      frontiers: list of node-id lists, the frontier of each step
      status: TREE_OK or TREE_E_PROB
      parent, tokens, q_row: flattened arrays of length T = m + 1 (or None)
    """
    root = dict(id=0, parent=-1, token=int(root_token), value=np.float32(1.0), depth=0, rank=0, q_row=-1)
    nodes = [root]
    frontier = [0]
    frontiers = []
    for s in range(depth):
        frontiers.append(list(frontier))
        layer = []
        for j, nid in enumerate(frontier):
            row = np.asarray(q_steps[s][j], dtype=np.float32)
            if not _row_ok(row):
                return dict(nodes=nodes, frontiers=frontiers, status=TREE_E_PROB, parent=None, tokens=None,
                            q_row=None)
            node = nodes[nid]
            node["q_row"] = s * k + j
            toks, probs = _top_tokens(row, k)
            for r in range(len(toks)):
                child = dict(id=len(nodes), parent=nid, token=int(toks[r]),
                             value=np.float32(np.float32(node["value"]) * np.float32(probs[r])),
                             depth=node["depth"] + 1, rank=r, q_row=-1)
                nodes.append(child)
                layer.append(child["id"])
        # next frontier: top-k of the new layer, value descending, then creation order
        ranked = sorted(layer, key=lambda i: (-float(nodes[i]["value"]), i))
        frontier = ranked[:k]
    draft = [n for n in nodes if n["id"] != 0]
    if m > len(draft):
        raise ValueError("m exceeds the generated nodes")
    kept = sorted(draft, key=lambda n: (-float(n["value"]), n["depth"], n["id"]))[:m]
    kept_ids = {n["id"] for n in kept}
    # flatten: depth, then parent position, then sibling rank
    pos = {0: 0}
    order = [0]
    for d in range(1, depth + 1):
        level = [n for n in kept if n["depth"] == d]
        level.sort(key=lambda n: (pos[n["parent"]], n["rank"]))
        for n in level:
            assert n["parent"] in kept_ids or n["parent"] == 0, "kept set not connected"
            pos[n["id"]] = len(order)
            order.append(n["id"])
    T = len(order)
    parent = np.full(T, -1, dtype=np.int32)
    tokens = np.zeros(T, dtype=np.int32)
    q_row = np.full(T, -1, dtype=np.int32)
    for p, nid in enumerate(order):
        n = nodes[nid]
        parent[p] = -1 if nid == 0 else pos[n["parent"]]
        tokens[p] = n["token"]
        q_row[p] = n["q_row"]
    return dict(nodes=nodes, frontiers=frontiers, status=TREE_OK, parent=parent, tokens=tokens, q_row=q_row,
                order=order)


def build(q_all, root_tokens, k, depth, m):
    """Batch form: q_all[s] is float32 [B][k][V] for step s.  Returns
    dict(parent [B][m+1], tokens [B][m+1], num_nodes [B], q_row [B][m+1],
    status [B], frontier [depth][B][k] (node ids, -1 padded), seqs)."""
    B = len(root_tokens)
    T = m + 1
    parent = np.full((B, T), -1, dtype=np.int32)
    tokens = np.full((B, T), -1, dtype=np.int32)
    q_row = np.full((B, T), -1, dtype=np.int32)
    num_nodes = np.zeros(B, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    frontier = np.full((depth, B, k), -1, dtype=np.int32)
    seqs = []
    for b in range(B):
        r = build_sequence([q_all[s][b] for s in range(depth)], int(root_tokens[b]), k, depth, m)
        seqs.append(r)
        status[b] = r["status"]
        for s, f in enumerate(r["frontiers"]):
            frontier[s, b, :len(f)] = f
        if r["status"] != TREE_OK:
            continue
        parent[b] = r["parent"]
        tokens[b] = r["tokens"]
        q_row[b] = r["q_row"]
        num_nodes[b] = T
    return dict(parent=parent, tokens=tokens, q_row=q_row, num_nodes=num_nodes, status=status,
                frontier=frontier, seqs=seqs)


def generated_nodes(k, depth):
    """Draft nodes generated by `depth` expansion steps of width k (closed
    form): k at step 0 (the root alone is expanded), k * k at every later step."""
    return k + (depth - 1) * k * k
