"""CPU oracle for draft-tree verification (test infrastructure only).

This module is the plain, slow, float64 definition of what the verification
step computes.  It exists to check the GPU library; it is not part of the
product path.  Only the test-suite, the smoke entry point and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP library.

Sources (web pages on EAGLE-style speculative decoding):

* [EAGLE article] the course.zhidx.com mirror of the Zhihu article on EAGLE,
  EAGLE-2, EAGLE-3 and DFlash; section 1.3 "Verification" (tree-wise
  verification, multi-round sibling sampling, Figure 1-6) and section 2.3
  "Flatten + Attention mask" (Figure 2-7).
* [Spec-decoding lesson] "投机解码与 EAGLE" (Speculative decoding and EAGLE),
  ai-engineering.com.cn; sections "Concept", "Exactness rule", "Tree-attention
  verification", "Expected speedup".

Readings where the pages are silent or garbled (each is listed with its reason
in the design notes of the repository):

* position 0 of every tree is the root (the last emitted token) and is a
  verify position; draft nodes are 1..T_b-1 with parent[i] < i;
* the tree mask is ancestor-or-self;
* attention scale 1/sqrt(D) unless given; query head h reads KV head
  floor(h / (Hq / Hkv));
* p = softmax(z / tau); tau <= 0 means greedy; ties break to the lowest index;
* sibling candidates are tested in increasing node index with the residual
  updated after each rejection; the proposal of the i-th sibling is q with the
  earlier siblings' tokens removed and renormalised when siblings were drawn
  without replacement, and q itself when drawn i.i.d.;
* the terminal draw is an inverse CDF in ascending token order;
* a draft token (position 1 .. T_b-1) outside [0, V), a stochastic sequence
  without draft probabilities, or a non-finite target logit in a row the walk
  reads (the row of every node it visits) marks the sequence invalid (count 0,
  outputs -1); rows of nodes the walk never reaches are not inspected, and the
  root's token (the last emitted token, never a candidate) is not read.

Parity is pinned by the tests under ``tests/test_oracle_*.py`` (closed forms,
the worked example trees and numbers the pages print, library routines for the
special cases, brute force).  No function here is unpinned.
"""
import math
import numpy as np

# Status codes (values are part of the library's interface contract).
TREE_OK = 0
TREE_E_ROOT = 1
TREE_E_PARENT = 2
TREE_E_COUNT = 3
TREE_E_TOKEN = 4
TREE_E_NONFINITE = 5
TREE_E_NOQ = 6
TREE_E_SYNC = 7      # device-side only (a cross-workgroup wait timed out)
TREE_E_CACHE = 8
TREE_E_PATH = 9

SIB_WITHOUT_REPLACEMENT = 0
SIB_IID = 1

EXEMPT_MARGIN = 1e-5


# --------------------------------------------------------------------------
# storage types
# --------------------------------------------------------------------------
def to_f64(arr, dtype):
    """Exact float64 value of stored data: 'bf16' (uint16 bit patterns) or 'f32'."""
    a = np.asarray(arr)
    if dtype == "bf16":
        bits = a.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# O1: flatten + tree attention mask
#   [EAGLE article, sec. 2.3 "Flatten + Attention mask"]: branches do not see
#   each other; each token sees only its ancestors on the tree.
#   [Spec-decoding lesson, "Tree-attention verification"]: every token attends
#   only to its ancestors in the tree.
# --------------------------------------------------------------------------
def check_tree(parent_row, T_b, T_max):
    """Status of one flattened tree: node count, root, topological parents."""
    if T_b < 1 or T_b > T_max:
        return TREE_E_COUNT
    if int(parent_row[0]) != -1:
        return TREE_E_ROOT
    for i in range(1, T_b):
        p = int(parent_row[i])
        if p < 0 or p >= i:
            return TREE_E_PARENT
    return TREE_OK


def ancestors(parent_row, i):
    """Ancestor-or-self set of node i, found by walking parent pointers."""
    out = []
    j = i
    while j != -1:
        out.append(j)
        j = int(parent_row[j])
    return out


def tree_mask(parent, num_nodes, T_max):
    """Ancestor-or-self mask of every sequence.

    Returns (anc_bool [B][T_max][T_max], anc_bits uint64 [B][T_max][W],
    depth int32 [B][T_max], status int32 [B]).  Bit j of word (j // 64) of
    row i is set iff node j is node i or one of its ancestors.  Rows and
    columns >= T_b, and every row of an invalid tree, are zero.
    """
    parent = np.asarray(parent)
    B = parent.shape[0]
    W = (T_max + 63) // 64
    anc = np.zeros((B, T_max, T_max), dtype=bool)
    depth = np.zeros((B, T_max), dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        T_b = int(num_nodes[b])
        status[b] = check_tree(parent[b], T_b, T_max)
        if status[b] != TREE_OK:
            continue
        for i in range(T_b):
            a = ancestors(parent[b], i)
            anc[b, i, a] = True
            depth[b, i] = len(a) - 1
    bits = np.zeros((B, T_max, W), dtype=np.uint64)
    for b in range(B):
        for i in range(T_max):
            for j in np.nonzero(anc[b, i])[0]:
                bits[b, i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return anc, bits, depth, status


# --------------------------------------------------------------------------
# O2: tree attention over the KV prefix plus tree ancestors
#   [EAGLE article, sec. 1.3 "Verification"]: the target computes every draft
#   token's probability in one forward using tree attention.
#   [Spec-decoding lesson, "Tree-attention verification"]: one forward, one
#   matmul; the topology mask costs only a few extra KV entries.
# --------------------------------------------------------------------------
def tree_attention(q, k_new, v_new, k_cache, v_cache, prefix_len, anc, num_nodes, status,
                   dtype, scale=0.0, units=None):
    """Masked attention of every tree position, float64.

    q [B][T_max][Hq][D], k_new/v_new [B][T_max][Hkv][D], k_cache/v_cache
    [B][Hkv][L_max][D] in storage ``dtype``; ``anc`` is the boolean mask from
    :func:`tree_mask`.  Position i of sequence b, query head h, attends to the
    first L_b cache entries of KV head floor(h / G) and to the tree tokens j
    with anc[b][i][j]; softmax(scale * q.k) weights the values.  Rows i >= T_b
    and sequences with a non-zero status are zero.  ``units``: optional list
    of (b, h) pairs to compute (the rest stays zero).
    """
    B, T_max, Hq, D = q.shape
    Hkv = k_new.shape[2]
    G = Hq // Hkv
    s = float(np.float32(scale)) if scale > 0 else 1.0 / math.sqrt(D)
    out = np.zeros((B, T_max, Hq, D), dtype=np.float64)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(Hq)]
    by_b = {}
    for b, h in units:
        by_b.setdefault(b, []).append(h)
    for b, heads in by_b.items():
        if status[b] != TREE_OK:
            continue
        T_b = int(num_nodes[b])
        L_b = int(prefix_len[b])
        Q = to_f64(q[b, :T_b], dtype)             # T_b x Hq x D
        Kt = to_f64(k_new[b, :T_b], dtype)        # T_b x Hkv x D
        Vt = to_f64(v_new[b, :T_b], dtype)
        visible = np.concatenate([np.ones((T_b, L_b), dtype=bool), anc[b, :T_b, :T_b]], axis=1)
        kv_rows = {}   # KV head -> its keys and values, widened once for its query heads
        for h in heads:
            kv = h // G
            if kv not in kv_rows:
                Kp = to_f64(k_cache[b, kv, :L_b], dtype)   # L_b x D
                Vp = to_f64(v_cache[b, kv, :L_b], dtype)
                kv_rows = {kv: (np.concatenate([Kp, Kt[:, kv]], axis=0),    # (L_b + T_b) x D
                                np.concatenate([Vp, Vt[:, kv]], axis=0))}
            Kall, Vall = kv_rows[kv]
            S = s * (Q[:, h] @ Kall.T)                      # T_b x (L_b + T_b)
            S = np.where(visible, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            E = np.exp(S)
            out[b, :T_b, h] = (E @ Vall) / E.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# O3: per-node target distribution
#   [Spec-decoding lesson, "Concept"]: the target scores all K+1 positions in
#   one forward; its code applies the temperature before the softmax.
#   [Spec-decoding lesson, "Exactness rule"], greedy case: compare with
#   argmax(p) only.
# --------------------------------------------------------------------------
def target_distribution(z, tau):
    """p = softmax(z / tau) in float64 (max-subtracted)."""
    z = np.asarray(z, dtype=np.float64)
    t = float(np.float32(tau))
    e = np.exp((z - z.max()) / t)
    return e / e.sum()


def argmax_lowest(z):
    """Index of the largest entry; the lowest such index on ties."""
    z = np.asarray(z)
    m = z.max()
    return int(np.nonzero(z == m)[0][0])


def inverse_cdf(P, u):
    """Smallest v with sum_{w<=v} P(w) > u; if rounding leaves none, the
    largest v with P(v) > 0.  Returns (v, margin) where margin is the distance
    of u to the CDF boundaries F(v-1), F(v) (F(-1) = 0 is exact and ignored).
    """
    F = np.cumsum(P)
    idx = np.nonzero(F > u)[0]
    if idx.size == 0:
        v = int(np.nonzero(P > 0)[0][-1])
    else:
        v = int(idx[0])
    hi = F[v] - u
    margin = abs(hi)
    if v > 0:
        margin = min(margin, abs(u - F[v - 1]))
    return v, float(margin)


# --------------------------------------------------------------------------
# O4: recursive accept / reject walk over the tree
#   [Spec-decoding lesson, "Exactness rule"]: accept x if r < p(x)/q(x); else
#   sample from (p - q)+ / ||(p - q)+||_1 and stop; greedy: accept iff
#   argmax(p) == x, else emit argmax(p) and stop.
#   [Spec-decoding lesson, "Concept"]: when every draft token is accepted, one
#   bonus token is sampled from p at the last position.
#   [EAGLE article, sec. 1.3 "Verification", Figure 1-6]: with k candidates at
#   one position, a rejected candidate is not the end: the next candidate is
#   tried with the corrected distribution, and only when all k are rejected is
#   the correction sampled; this is applied recursively at every node.
# --------------------------------------------------------------------------
def accept_walk(parent_row, tokens_row, T_b, zrow, qrow, tau, u_accept_row, u_sample_row,
                sibling_mode=SIB_WITHOUT_REPLACEMENT, reject_nonfinite=False):
    """Walk one verified tree from the root.

    ``zrow(n)`` returns the float64 target logits of node n (the target's
    distribution for the token after n); ``qrow(n)`` the float64 draft
    distribution node n's children were drawn from.  Returns a dict with
    ``nodes`` (accepted nodes, root excluded), ``emitted`` (their tokens plus
    the final correction / bonus token), ``count``, ``passes`` (vocabulary
    passes: one per rejection, one per bonus draw), ``decisions`` (list of
    (kind, node, margin)) and ``exempt_at`` (number of accepted nodes fixed
    before the first decision whose margin is below EXEMPT_MARGIN, or None).
    With ``reject_nonfinite`` (the input rule of ``spec_accept``), a visited
    node whose row holds a NaN or an infinity stops the walk, which returns
    ``{"nonfinite": True, "node": n}`` instead; without it a -inf logit is
    simply a token of target probability 0.
    """
    children = {n: [] for n in range(T_b)}
    for i in range(1, T_b):
        children[int(parent_row[i])].append(i)   # increasing index order
    greedy = not (float(np.float32(tau)) > 0.0)   # tau <= 0 (or NaN) selects greedy
    path, decisions = [], []
    passes = 0
    exempt_at = None
    n = 0
    while True:
        C = children[n]
        z = zrow(n)
        if reject_nonfinite and not np.all(np.isfinite(z)):
            return dict(nonfinite=True, node=n)
        if greedy:
            a = argmax_lowest(z)
            match = [c for c in C if int(tokens_row[c]) == a]
            if match:
                path.append(match[0])
                n = match[0]
                continue
            emitted = a
            break
        P = target_distribution(z, tau)
        Q = qrow(n) if C else None
        removed = []
        accepted = None
        for c in C:
            x = int(tokens_row[c])
            if sibling_mode == SIB_WITHOUT_REPLACEMENT:
                keep = np.ones(Q.size, dtype=bool)
                keep[removed] = False
                qi = np.where(keep, Q, 0.0)
                qi = qi / qi.sum()
            else:
                qi = Q
            if qi[x] > 0:
                ratio = P[x] / qi[x]
            else:
                ratio = math.inf if P[x] > 0 else 0.0
            u = float(u_accept_row[c])
            margin = abs(u - ratio) if math.isfinite(ratio) else math.inf
            decisions.append(("test", c, margin))
            if margin < EXEMPT_MARGIN and exempt_at is None:
                exempt_at = len(path)
            if u < ratio:
                accepted = c
                break
            R = np.maximum(0.0, P - qi)
            Z = R.sum()
            passes += 1
            if Z > 0:
                P = R / Z
            removed.append(x)
        if accepted is not None:
            path.append(accepted)
            n = accepted
            continue
        if not C:
            passes += 1          # bonus draw reads the row once more
        y, margin = inverse_cdf(P, float(u_sample_row[n]))
        decisions.append(("draw", n, margin))
        if margin < EXEMPT_MARGIN and exempt_at is None:
            exempt_at = len(path)
        emitted = y
        break
    return dict(nodes=path, emitted=[int(tokens_row[c]) for c in path] + [int(emitted)],
                count=len(path) + 1, passes=passes, decisions=decisions, exempt_at=exempt_at)


def spec_accept(parent, num_nodes, tokens, target_logits, logit_dtype, q_probs, temperature,
                u_accept, u_sample, status_in, sibling_mode=SIB_WITHOUT_REPLACEMENT, seqs=None):
    """Accept step for every sequence (or the listed ``seqs``).

    Returns dict with out_nodes [B][T_max], out_tokens [B][T_max] (-1 padded),
    out_count [B], status [B] and per-sequence ``walks`` (the accept_walk
    dicts, None for invalid or skipped sequences).
    """
    B, T_max = np.asarray(parent).shape
    V = target_logits.shape[2]
    out_nodes = np.full((B, T_max), -1, dtype=np.int32)
    out_tokens = np.full((B, T_max), -1, dtype=np.int32)
    out_count = np.zeros(B, dtype=np.int32)
    status = np.array(status_in, dtype=np.int32).copy()
    walks = [None] * B
    for b in (range(B) if seqs is None else seqs):
        if status[b] != TREE_OK:
            continue
        T_b = int(num_nodes[b])
        tk = np.asarray(tokens[b, 1:T_b], dtype=np.int64)   # draft tokens; the root's is not a candidate
        if np.any(tk < 0) or np.any(tk >= V):
            status[b] = TREE_E_TOKEN
            continue
        if q_probs is None and float(np.float32(temperature[b])) > 0.0:
            status[b] = TREE_E_NOQ      # stochastic verification needs the draft distribution
            continue
        w = accept_walk(parent[b], tokens[b], T_b,
                        lambda n, b=b: to_f64(target_logits[b, n], logit_dtype),
                        (lambda n, b=b: np.asarray(q_probs[b, n], dtype=np.float64))
                        if q_probs is not None else None,
                        float(temperature[b]), u_accept[b], u_sample[b], sibling_mode,
                        reject_nonfinite=True)
        if w.get("nonfinite"):
            status[b] = TREE_E_NONFINITE   # a row the walk read holds a NaN or an infinity
            continue
        walks[b] = w
        out_nodes[b, :len(w["nodes"])] = w["nodes"]
        out_tokens[b, :w["count"]] = w["emitted"]
        out_count[b] = w["count"]
    return dict(out_nodes=out_nodes, out_tokens=out_tokens, out_count=out_count, status=status,
                walks=walks)


# --------------------------------------------------------------------------
# Commit of the accepted path
#   [EAGLE article, sec. 1.3 "Verification"]: after verification the accepted
#   tokens and their features are kept and drafting continues from them.
#   [Spec-decoding lesson, "Concept"]: the accepted tokens extend the output;
#   the correction / bonus token is the next position to run the target on.
# Reading: the verified positions whose key/value rows enter the cache are the
# root (the last emitted token, verified in this pass) and the accepted nodes,
# in path order; the emitted token is the next root, so its rows come from
# the next forward pass.
# --------------------------------------------------------------------------
def commit_accepted(k_new, v_new, k_cache, v_cache, prefix_len, num_nodes, status_in, out_nodes,
                    out_count, feat_in=None):
    """Append the root's and the accepted nodes' K/V rows to the caches.

    k_new, v_new [B][T_max][Hkv][D]; k_cache, v_cache [B][Hkv][L_max][D] (any
    element type, copied bit for bit); out_nodes [B][T_max], out_count [B] as
    produced by spec_accept.  For a valid sequence with count c >= 1 the rows
    of positions [0, out_nodes[b][0], ..., out_nodes[b][c-2]] go to cache rows
    L_b .. L_b + c - 1 of every KV head and the new length is L_b + c; if that
    exceeds L_max the sequence gets TREE_E_CACHE, and if c > T_b or a path
    entry lies outside [1, T_b) it gets TREE_E_PATH; then nothing is written.
    feat_in [B][T_max][F] (optional): the same positions' rows go to rows
    0 .. c-1 of feat_out (other rows zero).
    Returns dict(k_cache, v_cache, prefix_len, status, feat_out) (copies).
    """
    k_cache = np.array(k_cache, copy=True)
    v_cache = np.array(v_cache, copy=True)
    B = k_cache.shape[0]
    L_max = k_cache.shape[2]
    new_len = np.array(prefix_len, dtype=np.int32).copy()
    status = np.array(status_in, dtype=np.int32).copy()
    feat_out = None if feat_in is None else np.zeros_like(feat_in)
    for b in range(B):
        c = int(out_count[b])
        if status[b] != TREE_OK or c < 1:
            continue
        L = int(prefix_len[b])
        T_b = int(num_nodes[b])
        positions = [0] + [int(out_nodes[b][i]) for i in range(c - 1)] if c <= T_b else None
        if positions is None or any(n < 1 or n >= T_b for n in positions[1:]):
            status[b] = TREE_E_PATH
            continue
        if L < 0 or L + c > L_max:
            status[b] = TREE_E_CACHE
            continue
        for i, n in enumerate(positions):
            k_cache[b, :, L + i, :] = k_new[b, n, :, :]
            v_cache[b, :, L + i, :] = v_new[b, n, :, :]
            if feat_out is not None:
                feat_out[b, i] = feat_in[b, n]
        new_len[b] = L + c
    return dict(k_cache=k_cache, v_cache=v_cache, prefix_len=new_len, status=status, feat_out=feat_out)


def verify_step(inst, sibling_mode=None, attn_units=None, accept_seqs=None):
    """Mask, attention and accept for one synthetic instance (float64)."""
    mode = sibling_mode
    if mode is None:
        mode = SIB_IID if inst.sibling_mode == "iid" else SIB_WITHOUT_REPLACEMENT
    anc, bits, depth, status = tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    out = None
    if inst.q is not None:
        out = tree_attention(inst.q, inst.k_new, inst.v_new, inst.k_cache, inst.v_cache,
                             inst.prefix_len, anc, inst.num_nodes, status, inst.dtype,
                             units=attn_units)
    acc = None
    if inst.target_logits is not None:
        acc = spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits,
                          inst.logit_dtype, inst.q_probs, inst.temperature, inst.u_accept,
                          inst.u_sample, status, mode, seqs=accept_seqs)
    return dict(anc=anc, anc_bits=bits, depth=depth, status=status, attn=out, accept=acc)
