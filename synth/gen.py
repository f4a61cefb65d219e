"""Seeded instance generation (NumPy Philox streams, host memory).

Recipe (one instance per (spec, seed)):

* ``SeedSequence([cfg_id, seed]).spawn(6)`` gives six independent Philox streams:
  tree shape, tree-token Q/K/V, KV cache, logits, draft draws, uniforms; the
  per-sequence ones (Q/K/V, cache, logits, draft draws) have one child stream
  per sequence.
* Tree: nodes at depth d+1 take a parent drawn uniformly from the depth-d nodes;
  nodes are numbered by depth, then parent, then draw order, so ``parent[i] < i``
  and siblings are contiguous in the order they were drafted.
* Logits: draft logits ``z_q ~ N(0, draft_std^2)`` per (sequence, node, token);
  target logits ``z_p = z_q + N(0, sigma^2)``, stored in ``logit_dtype``.
* Draft distribution (synthetic drafter): ``q = softmax(z_q / tau)`` in float64,
  stored float32; for a greedy sequence (tau = 0) the row holds softmax(z_q).
* Draft tokens: a node's children are drawn one after another from the stored
  q row of that node, without replacement ("wor") or i.i.d. ("iid"); for a
  greedy sequence they are the top-k of z_q (ties to the lowest index).  The root
  token is uniform over the vocabulary.
* Attention inputs q, k_new, v_new, k_cache, v_cache ~ N(0, 1), cast to ``dtype``;
  with ``qk_std`` = s the queries and keys are N(0, s^2) instead (score spread
  s^2 in natural units: a peaked softmax, as in a trained target's forward).
* ``plant`` = g (optional): every query row (sequence, position t < T_b, query
  head) gets one dominant key.  From its own Philox stream, each row picks
  the key of its own tree node, of its parent node (t > 0), or a uniform
  prefix key (L_b > 0), each allowed choice equally likely, and adds
  gamma * key to the query with gamma = g * qk_std^2 * sqrt(D) / |key|^2, so
  that this key's scaled score exceeds the random part by g * qk_std^2.
* Uniforms ``u_accept``, ``u_sample`` ~ U[0, 1) float32.

Padding rows (node index >= T_b) are filled too (random values, parent -1,
token 0); correct consumers never read them.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np


def bf16_bits_from_f32(x):
    """Round float32 to bfloat16 (nearest-even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32)
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        flat_out[s:s + step] = r.astype(np.uint16)
    return out


def f32_from_bf16_bits(b):
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Instance:
    spec: dict
    B: int
    T_max: int
    V: int
    Hq: int
    Hkv: int
    D: int
    L_max: int
    dtype: str
    logit_dtype: str
    sibling_mode: str
    parent: np.ndarray          # [B][T_max] int32
    num_nodes: np.ndarray       # [B] int32
    tokens: np.ndarray          # [B][T_max] int32
    prefix_len: np.ndarray      # [B] int32
    temperature: np.ndarray     # [B] float32
    q: np.ndarray = None        # [B][T_max][Hq][D]  (uint16 bf16 bits or float32)
    k_new: np.ndarray = None    # [B][T_max][Hkv][D]
    v_new: np.ndarray = None    # [B][T_max][Hkv][D]
    k_cache: np.ndarray = None  # [B][Hkv][L_max][D]
    v_cache: np.ndarray = None  # [B][Hkv][L_max][D]
    target_logits: np.ndarray = None  # [B][T_max][V] (uint16 bf16 bits or float32)
    q_probs: np.ndarray = None  # [B][T_max][V] float32
    u_accept: np.ndarray = None  # [B][T_max] float32
    u_sample: np.ndarray = None  # [B][T_max] float32
    extra: dict = field(default_factory=dict)


def tree_from_widths(widths, rng):
    """Parent array (root at 0) of a tree with ``widths[d]`` nodes at depth d+1.

    Each depth-(d+1) node picks its parent uniformly among the depth-d nodes;
    nodes are then numbered by depth, then parent index, then draw order.
    """
    parent = [-1]
    prev = [0]
    for w in widths:
        picks = rng.integers(0, len(prev), size=int(w))
        order = np.argsort(picks, kind="stable")
        cur = []
        for j in order:
            cur.append(len(parent))
            parent.append(prev[int(picks[j])])
        prev = cur
    return np.asarray(parent, dtype=np.int32)


def random_tree_widths(rng, depth_lo, depth_hi, width_lo, width_hi, n_lo, n_hi):
    """Per-depth widths drawn uniformly, resampled until the node count fits."""
    for _ in range(100000):
        depth = int(rng.integers(depth_lo, depth_hi + 1))
        widths = rng.integers(width_lo, width_hi + 1, size=depth)
        if n_lo <= int(widths.sum()) <= n_hi:
            return [int(w) for w in widths]
    raise RuntimeError("could not draw a tree of the requested size")


def _normal(rng, shape, std, out_dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if out_dtype == "bf16":
        return bf16_bits_from_f32(x)
    return x


def _per_seq(value, B, rng):
    if isinstance(value, (list, np.ndarray)):
        assert len(value) == B
        return list(value)
    if isinstance(value, tuple) and value[0] == "choice":
        opts = value[1]
        return [opts[int(i)] for i in rng.integers(0, len(opts), size=B)]
    return [value] * B


def _draw_children(qrow64, k, mode, rng):
    """k draft tokens from one q row (inverse CDF on the float64 row)."""
    w = qrow64.copy()
    out = []
    for _ in range(k):
        c = np.cumsum(w)
        u = rng.random()
        y = int(np.searchsorted(c, u * c[-1], side="right"))
        y = min(y, w.size - 1)
        while w[y] <= 0.0 and y > 0:   # never land on a zero-mass token
            y -= 1
        out.append(y)
        if mode == "wor":
            w[y] = 0.0
    return out


def _plant_keys(inst, b, Tb, gain, qk_std, rng):
    """Give every query row of sequence b (positions t < Tb) one dominant key
    (see the module docstring): its own tree node's key, its parent's, or a
    prefix key."""
    Lb = int(inst.prefix_len[b])
    G = inst.Hq // inst.Hkv
    D = inst.D
    widen = (lambda a: f32_from_bf16_bits(a)) if inst.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    q = widen(inst.q[b]).copy()
    k_new = widen(inst.k_new[b])
    k_cache = widen(inst.k_cache[b])
    for t in range(Tb):
        for h in range(inst.Hq):
            kv = h // G
            choices = ["self"] + (["parent"] if t > 0 else []) + (["prefix"] if Lb > 0 else [])
            pick = choices[int(rng.integers(0, len(choices)))]
            if pick == "self":
                key = k_new[t, kv]
            elif pick == "parent":
                key = k_new[int(inst.parent[b, t]), kv]
            else:
                key = k_cache[kv, int(rng.integers(0, Lb))]
            n2 = float(np.dot(key.astype(np.float64), key.astype(np.float64)))
            gamma = gain * qk_std * qk_std * np.sqrt(D) / max(n2, 1e-30)
            q[t, h] = q[t, h] + np.float32(gamma) * key
    inst.q[b] = bf16_bits_from_f32(q) if inst.dtype == "bf16" else q


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


def make_instance(spec, seed=0, with_attn=True, with_accept=True):
    """Build one seeded instance of ``spec`` (see :mod:`synth.configs`).

    Per-sequence data come from child streams of each Philox stream (one child
    per sequence), so sequences are generated in parallel threads and the
    result does not depend on the thread count.
    """
    s = dict(spec)
    B, Hq, Hkv, D, V = s["B"], s["Hq"], s["Hkv"], s["D"], s["V"]
    cfg_id = int(s.get("cfg_id", 0))
    ss = np.random.SeedSequence([cfg_id, int(seed)])
    s_tree, s_qkv, s_cache, s_logits, s_draft, s_unif = ss.spawn(6)
    r_tree = np.random.Generator(np.random.Philox(s_tree))
    r_unif = np.random.Generator(np.random.Philox(s_unif))
    child = lambda sq: [np.random.Generator(np.random.Philox(c)) for c in sq.spawn(B)]
    r_qkv, r_cache, r_logits, r_draft = child(s_qkv), child(s_cache), child(s_logits), child(s_draft)

    # ---- tree shapes
    kind = s["tree"][0]
    parents = []
    for b in range(B):
        if kind == "widths":
            parents.append(tree_from_widths(s["tree"][1], r_tree))
        elif kind == "chain":
            n = int(s["tree"][1])
            parents.append(np.arange(-1, n, dtype=np.int32))
        elif kind == "dynamic":
            widths = random_tree_widths(r_tree, *s["tree"][1:])
            parents.append(tree_from_widths(widths, r_tree))
        elif kind == "explicit":
            parents.append(np.asarray(s["tree"][1][b], dtype=np.int32))
        else:
            raise ValueError(kind)
    num_nodes = np.array([len(p) for p in parents], dtype=np.int32)
    T_max = int(s.get("T_max", num_nodes.max()))
    assert T_max >= num_nodes.max()
    parent = np.full((B, T_max), -1, dtype=np.int32)
    for b, p in enumerate(parents):
        parent[b, :len(p)] = p

    taus = np.asarray(_per_seq(s["tau"], B, r_tree), dtype=np.float32)
    pl = s["prefix_len"]
    prefix_len = np.asarray(pl if isinstance(pl, (list, tuple, np.ndarray)) else [pl] * B,
                            dtype=np.int32)
    L_max = int(s.get("L_max", max(1, int(prefix_len.max()))))
    dtype = s["dtype"]
    logit_dtype = s["logit_dtype"]
    mode = s.get("sibling_mode", "wor")

    inst = Instance(spec=s, B=B, T_max=T_max, V=V, Hq=Hq, Hkv=Hkv, D=D, L_max=L_max,
                    dtype=dtype, logit_dtype=logit_dtype, sibling_mode=mode,
                    parent=parent, num_nodes=num_nodes,
                    tokens=np.zeros((B, T_max), dtype=np.int32),
                    prefix_len=prefix_len, temperature=taus)
    store = np.uint16 if dtype == "bf16" else np.float32
    if with_attn:
        inst.q = np.empty((B, T_max, Hq, D), dtype=store)
        inst.k_new = np.empty((B, T_max, Hkv, D), dtype=store)
        inst.v_new = np.empty((B, T_max, Hkv, D), dtype=store)
        inst.k_cache = np.empty((B, Hkv, L_max, D), dtype=store)
        inst.v_cache = np.empty((B, Hkv, L_max, D), dtype=store)
    if with_accept:
        inst.target_logits = np.empty((B, T_max, V),
                                      dtype=np.uint16 if logit_dtype == "bf16" else np.float32)
        inst.q_probs = np.empty((B, T_max, V), dtype=np.float32)
    tokens = np.zeros((B, T_max), dtype=np.int32)
    draft_std = float(s.get("draft_std", 3.0))
    sigma = float(s.get("sigma", 1.0))
    qk_std = float(s.get("qk_std", 1.0))
    plant = s.get("plant")
    r_plant = child(np.random.SeedSequence([cfg_id, int(seed), 7])) if plant else None

    def one_sequence(b):
        # ---- attention inputs
        if with_attn:
            inst.q[b] = _normal(r_qkv[b], (T_max, Hq, D), qk_std, dtype)
            inst.k_new[b] = _normal(r_qkv[b], (T_max, Hkv, D), qk_std, dtype)
            inst.v_new[b] = _normal(r_qkv[b], (T_max, Hkv, D), 1.0, dtype)
            inst.k_cache[b] = _normal(r_cache[b], (Hkv, L_max, D), qk_std, dtype)
            inst.v_cache[b] = _normal(r_cache[b], (Hkv, L_max, D), 1.0, dtype)
            if plant:
                _plant_keys(inst, b, int(num_nodes[b]), float(plant), qk_std, r_plant[b])
        Tb = int(num_nodes[b])
        rd = r_draft[b]
        if not with_accept:
            # no logits: draft tokens are uniform (only the tree shape matters)
            tokens[b, :Tb] = rd.integers(0, V, size=Tb)
            return
        # ---- logits, draft distribution, draft tokens
        rl = r_logits[b]
        zq = rl.standard_normal(size=(T_max, V), dtype=np.float32) * np.float32(draft_std)
        zp = zq + rl.standard_normal(size=(T_max, V), dtype=np.float32) * np.float32(sigma)
        tau = float(taus[b])
        t_eff = tau if tau > 0 else 1.0
        z64 = zq.astype(np.float64) / t_eff
        z64 -= z64.max(axis=1, keepdims=True)
        np.exp(z64, out=z64)
        z64 /= z64.sum(axis=1, keepdims=True)
        q32 = z64.astype(np.float32)
        del z64
        inst.target_logits[b] = bf16_bits_from_f32(zp) if logit_dtype == "bf16" else zp
        inst.q_probs[b] = q32
        tokens[b, 0] = int(rd.integers(0, V))
        par = parent[b, :Tb]
        for n in range(Tb):
            kids = np.nonzero(par == n)[0]
            if kids.size == 0:
                continue
            if tau > 0:
                drawn = _draw_children(q32[n].astype(np.float64), kids.size, mode, rd)
            else:
                drawn = [int(i) for i in np.argsort(-zq[n], kind="stable")[:kids.size]]
            tokens[b, kids] = drawn

    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(one_sequence, range(B)))
    inst.tokens = tokens
    inst.u_accept = r_unif.random(size=(B, T_max), dtype=np.float32)
    inst.u_sample = r_unif.random(size=(B, T_max), dtype=np.float32)
    return inst


def make_draft_rows(B, k, depth, V, seed=0, draft_std=3.0, tie_step=None, cfg_id=900):
    """Synthetic drafter output for the tree builder: for each expansion step
    s, a float32 array [B][k][V] whose row j is the probability row the drafter
    gives for frontier entry j, ``softmax(N(0, draft_std^2))`` computed in
    float64.  The rows do not depend on which node they end up attached to
    (that is decided by the builder).  With ``tie_step`` set, probabilities are
    rounded down to multiples of ``tie_step`` so that equal values (ties) are
    common.  Seeded by ``SeedSequence([cfg_id, seed])``, one Philox stream per
    step."""
    streams = np.random.SeedSequence([cfg_id, int(seed)]).spawn(depth)
    out = []
    for s in range(depth):
        rng = np.random.Generator(np.random.Philox(streams[s]))
        z = rng.standard_normal((B, k, V)) * draft_std
        z -= z.max(axis=2, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=2, keepdims=True)
        if tie_step is not None:
            p = np.floor(p / tie_step) * tie_step
        out.append(p.astype(np.float32))
    return out


def make_head_inputs(N, d, r, n, seed=0, quantized=True, with_W=True, cfg_id=910):
    """Inputs of the two-stage draft head: h [N][d], B [r][d], A_sh [n][r],
    W [n][d] as bf16 bit patterns (uint16) and a shuffle perm [n] (int32).
    With ``quantized`` every value is a multiple of 1/8 in [-1, 1], so float32
    sums of their products are exact (and so is u = B h at these sizes);
    otherwise N(0, 1) for h and N(0, 1/d), N(0, 1/r) for the factors and W.
    Seeded by ``SeedSequence([cfg_id, seed])``: one Philox stream per tensor."""
    ss = np.random.SeedSequence([cfg_id, int(seed)]).spawn(5)
    g = [np.random.Generator(np.random.Philox(x)) for x in ss]

    def draw(rng, shape, std):
        if quantized:
            return (rng.integers(-8, 9, size=shape) / 8.0).astype(np.float32)
        return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std))

    h = bf16_bits_from_f32(draw(g[0], (N, d), 1.0))
    B = bf16_bits_from_f32(draw(g[1], (r, d), 1.0 / np.sqrt(d)))
    A_sh = bf16_bits_from_f32(draw(g[2], (n, r), 1.0 / np.sqrt(r)))
    perm = g[3].permutation(n).astype(np.int32)
    W = bf16_bits_from_f32(draw(g[4], (n, d), 1.0 / np.sqrt(d))) if with_W else None
    return dict(h=h, B=B, A_sh=A_sh, perm=perm, W=W)
