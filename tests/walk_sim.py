"""Tiny synthetic 'models' for statistical tests of the accept walk.

A model is a table of target distributions p(. | context) and draft
distributions q(. | context) keyed by the token path from the root.  The
drafter (test side) draws sibling tokens from q, without replacement or i.i.d.;
the walk under test sees log p as its target logits at temperature 1.
"""
import numpy as np


class PathModel:
    def __init__(self, V, seed, conc_p=1.0, conc_q=1.0, fixed=None):
        self.V = V
        self.seed = seed
        self.conc_p, self.conc_q = conc_p, conc_q
        self.fixed = fixed          # optional (p, q) used for every context
        self.cache = {}

    def pq(self, ctx):
        ctx = tuple(ctx)
        if self.fixed is not None:
            return self.fixed
        if ctx not in self.cache:
            r = np.random.default_rng([self.seed, len(ctx)] + list(ctx))
            p = r.dirichlet(np.full(self.V, self.conc_p))
            q = r.dirichlet(np.full(self.V, self.conc_q))
            self.cache[ctx] = (p, q)
        return self.cache[ctx]


def draw_siblings(q, k, mode, rng):
    w = np.array(q, dtype=np.float64)
    out = []
    for _ in range(k):
        c = np.cumsum(w)
        y = int(np.searchsorted(c, rng.random() * c[-1], side="right"))
        y = min(y, w.size - 1)
        while w[y] <= 0:
            y -= 1
        out.append(y)
        if mode == "wor":
            w[y] = 0.0
    return out


def build_tree(model, ctx0, widths_per_depth, mode, rng):
    """Draft a tree: every node at depth d gets widths_per_depth[d] children.

    Returns parent, tokens, contexts (token path from the root, root excluded).
    """
    parent, tokens, ctxs = [-1], [-1], [tuple(ctx0)]
    frontier = [0]
    for k in widths_per_depth:
        nxt = []
        for n in frontier:
            _, q = model.pq(ctxs[n])
            for t in draw_siblings(q, k, mode, rng):
                parent.append(n)
                tokens.append(t)
                ctxs.append(ctxs[n] + (t,))
                nxt.append(len(parent) - 1)
        frontier = nxt
    tokens[0] = 0
    return np.array(parent), np.array(tokens), ctxs


def run_walk(oracle, model, parent, tokens, ctxs, rng, mode_const, tau=1.0):
    T = len(parent)
    with np.errstate(divide="ignore"):
        zrow = lambda n: np.log(model.pq(ctxs[n])[0])
    qrow = lambda n: model.pq(ctxs[n])[1]
    ua = rng.random(T)
    us = rng.random(T)
    return oracle.accept_walk(parent, tokens, T, zrow, qrow, tau, ua, us, mode_const)


def tv(counts, p):
    f = counts / counts.sum()
    return 0.5 * float(np.abs(f - p).sum())
