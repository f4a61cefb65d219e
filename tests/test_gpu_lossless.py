"""Losslessness of the GPU walk itself (sv_spec_accept), measured by sampling.

[Spec-decoding lesson] "Exactness rule" and its exercise: speculative
sampling must leave the law of the emitted tokens equal to the target's; the
exercise's check is a total-variation distance below 0.01 between the
sampled and the target distribution.  Here 100,000 independent trials run as
one batch of 100,000 sequences through one sv_spec_accept call: every trial
drafts its own tree from q (the drafter, on the host) with its own uniforms,
and the target logits are log p at temperature 1.  The first emitted token
must follow p at the root.  Cases: a chain, three i.i.d. siblings, three
siblings without replacement, a depth-3 tree; and the negative control the
oracle's pins use: siblings drawn without replacement but walked as if drawn
i.i.d. (the proposal update dropped) must show a clear bias, so the
statistic has the power to see a wrong rule.
"""
import numpy as np
import pytest

from gpu_util import need_gpu, say, sv_problem
from walk_sim import PathModel, build_tree, tv

pytestmark = pytest.mark.gpu

TRIALS = 100_000
NEG_P = np.array([0.106, 0.031, 0.533, 0.036, 0.011, 0.178, 0.049, 0.056])
NEG_Q = np.array([0.006, 0.157, 0.214, 0.047, 0.345, 0.043, 0.162, 0.026])


class _Batch:
    """One sequence per trial, in the layout the library takes."""

    def __init__(self, model, widths, draft_mode, walk_mode, seed, trials=TRIALS):
        rng = np.random.default_rng(seed)
        trees = [build_tree(model, (), widths, draft_mode, rng) for _ in range(trials)]
        T = max(len(t[0]) for t in trees)
        V = model.V
        self.B, self.T_max, self.V = trials, T, V
        self.parent = np.full((trials, T), -1, np.int32)
        self.tokens = np.zeros((trials, T), np.int32)
        self.num_nodes = np.zeros(trials, np.int32)
        ids = {}                                   # context -> row of the tables below
        row = np.zeros((trials, T), np.int64)      # padding positions use row 0 (never read)
        for b, (par, tok, ctxs) in enumerate(trees):
            n = len(par)
            self.parent[b, :n] = par
            self.tokens[b, :n] = tok
            self.num_nodes[b] = n
            row[b, :n] = [ids.setdefault(c, len(ids)) for c in ctxs]
        z_tab = np.zeros((len(ids), V), np.float32)
        q_tab = np.zeros((len(ids), V), np.float32)
        for c, i in ids.items():
            p, q = model.pq(c)
            with np.errstate(divide="ignore"):
                z_tab[i] = np.log(p)
            q_tab[i] = q
        self.target_logits = z_tab[row]
        self.q_probs = q_tab[row]
        self.logit_dtype = "f32"
        self.temperature = np.ones(trials, np.float32)
        self.u_accept = rng.random((trials, T), dtype=np.float32)
        self.u_sample = rng.random((trials, T), dtype=np.float32)
        self.sibling_mode = walk_mode
        self.p_root = model.pq(())[0]


def _first_token_tv(batch, label):
    say(f"lossless {label}: {batch.B} walks, T_max={batch.T_max}, V={batch.V}, walk mode {batch.sibling_mode}")
    dev = sv_problem(batch, with_attn=False)
    dev.mask_build()
    dev.spec_accept()
    res = dev.accept_results()
    assert (res["status"] == 0).all()
    first = res["out_tokens"][:, 0]
    assert ((first >= 0) & (first < batch.V)).all()
    d = tv(np.bincount(first, minlength=batch.V).astype(np.float64), batch.p_root)
    say(f"  TV(first token, p_root) = {d:.4f}")
    return d


@pytest.mark.parametrize("seed,widths,draft_mode,walk_mode", [
    (201, [1, 1, 1], "iid", "wor"),        # chain
    (202, [3], "iid", "iid"),              # i.i.d. siblings, k = 3
    (203, [3], "wor", "wor"),              # siblings without replacement, k = 3
    (204, [2, 2, 1], "wor", "wor"),        # depth-3 tree
])
def test_gpu_first_token_total_variation(seed, widths, draft_mode, walk_mode):
    need_gpu()
    model = PathModel(8, 5, conc_p=1.0, conc_q=1.0)
    b = _Batch(model, widths, draft_mode, walk_mode, seed)
    assert _first_token_tv(b, f"widths={widths} drafted {draft_mode}") < 0.01


def test_gpu_negative_control_sibling_rule():
    """Siblings drawn without replacement: walked with the proposal update the
    law is exact; walked as if i.i.d. it is biased (TV about 0.06 on the
    oracle's pin with the same distributions)."""
    need_gpu()
    model = PathModel(8, 0, fixed=(NEG_P, NEG_Q))
    good = _first_token_tv(_Batch(model, [3], "wor", "wor", 21), "negative control, right rule")
    bad = _first_token_tv(_Batch(model, [3], "wor", "iid", 21), "negative control, update dropped")
    assert good < 0.01
    assert bad > 0.03
