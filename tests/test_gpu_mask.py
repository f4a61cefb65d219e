"""GPU tree mask (sv_tree_mask_build) against the oracle: bit-exact masks,
depths and statuses on the five workload trees, random trees up to T_max =
256, single-node trees and malformed trees."""
import numpy as np
import pytest

from gpu_util import check_mask, need_gpu, say, sv_problem
from synth import CONFIGS, make_instance

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [c["name"] for c in CONFIGS])
def test_mask_workload_trees(cfg):
    need_gpu()
    spec = dict(next(c for c in CONFIGS if c["name"] == cfg))
    spec["V"] = 64
    inst = make_instance(spec, 0, with_attn=False, with_accept=False)
    say(f"mask {cfg} B={inst.B} T_max={inst.T_max}")
    dev = sv_problem(inst, with_attn=False, with_accept=False)
    dev.mask_build()
    st = check_mask(dev, inst)
    assert (st == 0).all()


class _Trees:
    def __init__(self, parents, T_max, counts=None):
        self.B = len(parents)
        self.T_max = T_max
        self.parent = np.full((self.B, T_max), -1, dtype=np.int32)
        for b, p in enumerate(parents):
            self.parent[b, :len(p)] = p
        self.num_nodes = np.array(counts if counts is not None else [len(p) for p in parents], dtype=np.int32)
        self.tokens = np.zeros((self.B, T_max), dtype=np.int32)


@pytest.mark.parametrize("T_max", [1, 7, 64, 65, 129, 200, 256])
def test_mask_random_trees(T_max):
    need_gpu()
    rng = np.random.default_rng(T_max)
    parents = []
    for b in range(9):
        T = int(rng.integers(1, T_max + 1)) if b else T_max
        p = [-1] + [int(rng.integers(0, i)) for i in range(1, T)]
        parents.append(p)
    parents.append([-1])
    src = _Trees(parents, T_max)
    say(f"mask random T_max={T_max}")
    dev = sv_problem(src, with_attn=False, with_accept=False)
    dev.mask_build()
    st = check_mask(dev, src)
    assert (st == 0).all()


def test_mask_malformed_trees():
    need_gpu()
    T = 6
    parents = [[-1, 0, 0, 1, 2, 3], [0, 0, 0, 1, 2, 3], [-1, 0, 2, 1, 2, 3], [-1, 0, 0, 7, 2, 3],
               [-1, 0, 0, 1, 2, 3], [-1, 0, 0, 1, 2, 3], [-1, -1, 0, 1, 2, 3], [-1, 0, 0, 1, 2, 3]]
    counts = [6, 6, 6, 6, 0, 7, -3, 3]
    src = _Trees(parents, T, counts)
    say("mask malformed")
    dev = sv_problem(src, with_attn=False, with_accept=False)
    dev.mask_build()
    st = check_mask(dev, src)
    assert st.tolist() == [0, 1, 2, 2, 3, 3, 3, 0]
