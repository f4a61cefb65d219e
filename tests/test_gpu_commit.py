"""GPU commit of the accepted path (sv_commit_accepted) against the oracle.

The commit is a copy, so caches, new lengths, statuses and feature rows must
match the oracle bit for bit.  Cases: after a real verification step (greedy
and stochastic sequences, ragged prefixes including 0), bf16 and fp32, head
dims 64 and 128, features of widths that are and are not multiples of 8,
a cache without room, path entries out of range, an invalid tree, and the
70B-shaped workload at full size.
"""
import numpy as np
import pytest

import oracle
from gpu_util import need_gpu, say, sv_problem
from synth import CONFIGS, make_instance

pytestmark = pytest.mark.gpu


def _spec(**kw):
    s = dict(cfg_id=600, B=6, Hq=8, Hkv=2, D=128, dtype="bf16", logit_dtype="bf16", prefix_len=[40, 0, 77, 5, 120, 9],
             tree=("dynamic", 1, 5, 1, 5, 1, 30), V=500, tau=("choice", [0.0, 0.8, 1.0]), sigma=0.5,
             draft_std=1.5, sibling_mode="wor", L_max=200)
    s.update(kw)
    return s


def _host(t, dtype):
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _run(inst, label, F=0, mutate=None):
    import torch
    say(f"commit {label} B={inst.B} Hkv={inst.Hkv} D={inst.D} L_max={inst.L_max} F={F}")
    dev = sv_problem(inst)
    dev.verify_step()
    if mutate:
        mutate(dev)
    feat_in = None
    if F:
        g = torch.Generator(device="cpu").manual_seed(F)
        host = torch.randn((inst.B, inst.T_max, F), generator=g)
        feat_in = host.to(torch.bfloat16 if inst.dtype == "bf16" else torch.float32).to(dev.k_new.device)
    dev.commit_args(feat_in)
    acc = dev.accept_results()
    k0, v0 = _host(dev.k_cache, inst.dtype), _host(dev.v_cache, inst.dtype)
    dev.commit_accepted()
    torch.cuda.synchronize()
    fin = None if feat_in is None else _host(feat_in, inst.dtype)
    ref = oracle.commit_accepted(_host(dev.k_new, inst.dtype), _host(dev.v_new, inst.dtype), k0, v0,
                                 inst.prefix_len, inst.num_nodes, acc["status"], acc["out_nodes"],
                                 acc["out_count"], fin)
    np.testing.assert_array_equal(dev.status.cpu().numpy(), ref["status"])
    np.testing.assert_array_equal(dev.prefix_len_out.cpu().numpy(), ref["prefix_len"])
    np.testing.assert_array_equal(_host(dev.k_cache, inst.dtype), ref["k_cache"])
    np.testing.assert_array_equal(_host(dev.v_cache, inst.dtype), ref["v_cache"])
    if F:
        np.testing.assert_array_equal(_host(dev.feat_out, inst.dtype), ref["feat_out"])
    return ref


@pytest.mark.parametrize("dtype,D,F", [("bf16", 128, 64), ("bf16", 64, 33), ("f32", 64, 0), ("f32", 128, 7)])
def test_commit_after_verification(dtype, D, F):
    need_gpu()
    inst = make_instance(_spec(dtype=dtype, D=D, logit_dtype=dtype), 1)
    ref = _run(inst, f"{dtype} D={D}", F)
    assert (ref["prefix_len"] > inst.prefix_len).any()


def test_commit_errors():
    need_gpu()
    inst = make_instance(_spec(B=5, prefix_len=[197, 3, 6, 2, 2], tree=("widths", [3, 3])), 2)

    def mutate(dev):
        import torch
        c = dev.out_count.cpu()
        n = dev.out_nodes.cpu()
        s = dev.status.cpu()
        c[0] = 5               # a valid path of 5 positions, but 197 + 5 > 200: no room
        n[0, :4] = torch.tensor([1, 2, 3, 4], dtype=n.dtype)
        s[2] = oracle.TREE_E_PARENT
        c[3], n[3, 0] = 2, 99  # path entry outside the tree
        c[4] = 40              # more positions than the tree has
        dev.out_count.copy_(c)
        dev.out_nodes.copy_(n)
        dev.status.copy_(s)
    ref = _run(inst, "errors", F=16, mutate=mutate)
    assert ref["status"].tolist()[:1] + ref["status"].tolist()[2:] == [
        oracle.TREE_E_CACHE, oracle.TREE_E_PARENT, oracle.TREE_E_PATH, oracle.TREE_E_PATH]


def test_commit_full_workload():
    need_gpu()
    spec = dict(next(c for c in CONFIGS if c["name"] == "tree64_llama70b_b32"))
    spec["L_max"] = spec["prefix_len"] + 128
    spec["V"] = 2000        # the vocabulary does not affect the commit
    inst = make_instance(spec, 0)
    _run(inst, "tree64_llama70b_b32 shape", F=256)
