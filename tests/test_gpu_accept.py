"""GPU accept / reject (sv_spec_accept) against the oracle's walk.

Accepted paths, emitted tokens, counts and vocabulary-pass counts must match
bit for bit up to the first decision whose oracle margin is below 1e-5 (the
exemption band); after it the GPU path must still be a valid tree path.
Cases: small vocabularies split over several workgroups (the cross-workgroup
residual passes), a vocabulary that is not a multiple of 8 (scalar loads),
fp32 and bf16 logits, greedy / stochastic / mixed temperatures, both sibling
modes, single-node trees, malformed inputs, and the five workloads at full
size.
"""
import numpy as np
import pytest

import oracle
from gpu_util import check_accept, check_path_valid, need_gpu, say, sv_problem
from synth import CONFIGS, make_instance

pytestmark = pytest.mark.gpu


def _spec(**kw):
    s = dict(cfg_id=200, B=6, Hq=4, Hkv=4, D=64, dtype="bf16", logit_dtype="bf16", prefix_len=8,
             tree=("dynamic", 1, 5, 1, 6, 1, 40), V=5000, tau=1.0, sigma=1.0, draft_std=3.0,
             sibling_mode="wor")
    s.update(kw)
    return s


def _mode(inst):
    return oracle.SIB_IID if inst.sibling_mode == "iid" else oracle.SIB_WITHOUT_REPLACEMENT


def _run(inst, label, mutate=None):
    say(f"accept {label} B={inst.B} T_max={inst.T_max} V={inst.V} tau={inst.temperature.tolist()[:8]}")
    dev = sv_problem(inst, with_attn=False)
    if mutate:
        mutate(dev)
    dev.mask_build()
    dev.spec_accept()
    res = dev.accept_results()
    _, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    ref = oracle.spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits,
                             inst.logit_dtype, inst.q_probs if not getattr(inst, "_no_q", False) else None,
                             inst.temperature, inst.u_accept, inst.u_sample, status, _mode(inst))
    exempt = check_accept(res, ref, label)
    for b in range(inst.B):
        if res["out_count"][b] > 0:
            check_path_valid(res, inst, b)
    return res, ref, exempt


SMALL = {
    "stochastic_wor_bf16": _spec(),
    "stochastic_iid_bf16": _spec(cfg_id=201, sibling_mode="iid"),
    "greedy_bf16": _spec(cfg_id=202, tau=0.0),
    "mixed_tau_bf16": _spec(cfg_id=203, B=9, tau=("choice", [0.0, 0.7, 1.0])),
    "stochastic_f32": _spec(cfg_id=204, logit_dtype="f32", V=3000),
    "greedy_f32": _spec(cfg_id=205, logit_dtype="f32", tau=0.0, V=3000),
    "odd_vocab_bf16": _spec(cfg_id=206, V=4097),
    "odd_vocab_f32_iid": _spec(cfg_id=207, V=2999, logit_dtype="f32", sibling_mode="iid"),
    "single_node_trees": _spec(cfg_id=208, tree=("chain", 0), tau=("choice", [0.0, 1.0])),
    "chain_stochastic": _spec(cfg_id=209, tree=("chain", 6), tau=0.8),
    "wide_tree_big_vocab": _spec(cfg_id=210, B=3, tree=("widths", [8, 16, 24]), V=40000, tau=0.7),
    "many_sequences": _spec(cfg_id=211, B=70, V=2048, tree=("dynamic", 1, 4, 1, 4, 1, 20)),
    "low_temperature": _spec(cfg_id=212, tau=0.3, sigma=0.3),
    "high_temperature": _spec(cfg_id=213, tau=2.0, sigma=2.0),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_accept_small(name):
    need_gpu()
    inst = make_instance(SMALL[name], 5, with_attn=False)
    _run(inst, name)


@pytest.mark.parametrize("seed", range(4))
def test_accept_fuzz(seed):
    need_gpu()
    rng = np.random.default_rng(seed)
    spec = _spec(cfg_id=300 + seed, B=int(rng.integers(1, 12)), V=int(rng.integers(50, 30000)),
                 logit_dtype=["bf16", "f32"][seed % 2], sibling_mode=["wor", "iid"][(seed // 2) % 2],
                 tau=("choice", [0.0, 0.5, 1.0, 1.5]),
                 tree=("dynamic", 1, 7, 1, 10, 1, 100))
    inst = make_instance(spec, seed, with_attn=False)
    _run(inst, f"fuzz{seed}")


def test_accept_malformed_inputs():
    need_gpu()
    inst = make_instance(_spec(cfg_id=220, B=8, tau=1.0, V=3000), 9, with_attn=False)
    # rows the clean walk never reads (neither the root, nor an accepted node)
    _, _, _, status0 = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    clean = oracle.spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits, "bf16",
                               inst.q_probs, inst.temperature, inst.u_accept, inst.u_sample, status0)
    visited7 = {0} | set(clean["walks"][7]["nodes"])
    unvisited7 = [n for n in range(int(inst.num_nodes[7])) if n not in visited7]
    assert unvisited7, "sequence 7 must have a node the walk skips"
    inst.parent[0, 1] = 3                         # tree error
    inst.tokens[1, 1] = inst.V                    # token out of range
    inst.tokens[2, 0] = -1                        # the root's token is never read
    bits = {"nan": 0x7FC0, "inf": 0x7F80, "-inf": 0xFF80}
    inst.target_logits[3, 0, 17] = bits["nan"]                       # the root row is always read
    inst.target_logits[4, int(inst.num_nodes[4]) - 1, 5] = bits["inf"]  # read only if visited
    inst.target_logits[5, 0, 4095 % inst.V] = bits["-inf"]
    # a non-finite value past the tree is never read
    if int(inst.num_nodes[6]) < inst.T_max:
        inst.target_logits[6, inst.T_max - 1, 3] = bits["nan"]
    inst.target_logits[7, unvisited7[-1], 11] = bits["nan"]          # a row the walk never reads
    res, ref, _ = _run(inst, "malformed")
    assert res["status"][:4].tolist() == [oracle.TREE_E_PARENT, oracle.TREE_E_TOKEN, oracle.TREE_OK,
                                          oracle.TREE_E_NONFINITE]
    np.testing.assert_array_equal(res["out_tokens"][2], clean["out_tokens"][2])
    assert res["status"][5] == oracle.TREE_E_NONFINITE
    assert res["status"][4] == ref["status"][4]
    assert res["status"][6] == 0 and res["status"][7] == 0
    np.testing.assert_array_equal(res["out_tokens"][7], clean["out_tokens"][7])


def test_accept_without_draft_probabilities():
    need_gpu()
    inst = make_instance(_spec(cfg_id=221, B=4, tau=[0.0, 1.0, 0.0, 0.5]), 1, with_attn=False)
    say("accept q=NULL")
    from eagle_tree_verification_attn_amd import make_accept_args
    dev = sv_problem(inst, with_attn=False)
    dev.q_probs = None
    dev.acc = make_accept_args(dev.logits, None, dev.temperature, dev.u_accept, dev.u_sample,
                               dev.out_tokens, dev.out_nodes, dev.out_count, dev.out_passes, 0)
    dev.mask_build()
    dev.spec_accept()
    res = dev.accept_results()
    assert res["status"].tolist() == [0, oracle.TREE_E_NOQ, 0, oracle.TREE_E_NOQ]
    inst._no_q = True
    _, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    ref = oracle.spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits, "bf16", None,
                             inst.temperature, inst.u_accept, inst.u_sample, status, seqs=[0, 2])
    for b in (0, 2):
        np.testing.assert_array_equal(res["out_tokens"][b], ref["out_tokens"][b])
        assert res["out_count"][b] == ref["out_count"][b]


def test_accept_repeatable():
    """Two runs give identical outputs (the cross-workgroup passes are ordered)."""
    need_gpu()
    inst = make_instance(_spec(cfg_id=222, B=16, V=20000, tau=0.9), 2, with_attn=False)
    say("accept repeat")
    dev = sv_problem(inst, with_attn=False)
    outs = []
    for _ in range(3):
        dev.mask_build()
        dev.spec_accept()
        outs.append(dev.accept_results())
    for o in outs[1:]:
        for k in ("out_nodes", "out_tokens", "out_count", "out_passes"):
            np.testing.assert_array_equal(o[k], outs[0][k])


@pytest.mark.parametrize("cfg", [c["name"] for c in CONFIGS])
def test_accept_full_workloads(cfg):
    need_gpu()
    spec = dict(next(c for c in CONFIGS if c["name"] == cfg))
    inst = make_instance(spec, 0, with_attn=False)
    res, ref, exempt = _run(inst, f"full {cfg}")
    say(f"  counts {res['out_count'].tolist()} passes {res['out_passes'].tolist()} exempt {exempt}")


def test_accept_on_two_streams_ordered_by_events():
    """Walks on two streams, each ordered after the other's previous walk by an
    event (the rule for walks on one device), give the results of serial calls."""
    need_gpu()
    import torch
    insts = [make_instance(_spec(cfg_id=223, B=16, V=20000, tau=0.9), s, with_attn=False) for s in (3, 4)]
    say("accept two streams with events")
    serial = []
    for inst in insts:
        dev = sv_problem(inst, with_attn=False)
        dev.mask_build()
        dev.spec_accept()
        serial.append(dev.accept_results())
    devs = [sv_problem(inst, with_attn=False) for inst in insts]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    done = None
    for r in range(4):
        i = r % 2
        s = streams[i]
        devs[i].mask_build(stream=s)
        if done is not None:
            s.wait_event(done)
        devs[i].spec_accept(stream=s)
        done = torch.cuda.Event()
        done.record(s)
    torch.cuda.synchronize()
    for i, dev in enumerate(devs):
        got = dev.accept_results()
        for k in ("out_nodes", "out_tokens", "out_count", "out_passes"):
            np.testing.assert_array_equal(got[k], serial[i][k])


def test_accept_gives_up_cleanly_when_waits_end_at_once():
    """With the exchange-wait bound at 0 ticks (SV_WALK_WAIT_TICKS=0) every
    wait that does not find its value at once gives up, as when a group's
    workgroups are not all resident together.  Every workgroup still ends.
    Each sequence is then either complete and equal to the oracle, or marked
    SV_TREE_E_SYNC with -1 / count 0 outputs (a sequence with its own data
    error keeps that status); once a group gives up at one of its sequences,
    its later sequences are marked too.  A call with the normal bound on the
    same buffers then gives the oracle's results."""
    need_gpu()
    import os
    spec = _spec(cfg_id=224, B=64, V=131072, tree=("widths", [2, 2]), tau=1.0)
    inst = make_instance(spec, 6, with_attn=False)
    inst.parent[40, 2] = 2                        # a data error of its own (parent not before the node)
    _, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    ref = oracle.spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits, "bf16",
                             inst.q_probs, inst.temperature, inst.u_accept, inst.u_sample, status)
    dev = sv_problem(inst, with_attn=False)
    say("accept give-up path: SV_WALK_WAIT_TICKS=0, B=64 V=131072 (2 sequences per group)")
    os.environ["SV_WALK_WAIT_TICKS"] = "0"
    try:
        dev.mask_build()
        dev.spec_accept()
        res = dev.accept_results()
    finally:
        os.environ.pop("SV_WALK_WAIT_TICKS", None)
    import torch
    B = inst.B
    ngroups = min(B, torch.cuda.get_device_properties(0).multi_processor_count // 8)   # 8 chunks of 16384
    st = res["status"]
    n_sync = int((st == oracle.TREE_E_SYNC).sum())
    say(f"  gave up on {n_sync} of {B} sequences")
    assert st[40] == oracle.TREE_E_PARENT
    for b in range(B):
        if st[b] == oracle.TREE_E_SYNC or b == 40:
            assert res["out_count"][b] == 0, b
            assert (res["out_nodes"][b] == -1).all() and (res["out_tokens"][b] == -1).all(), b
            assert res["out_passes"][b] == 0, b
            if st[b] == oracle.TREE_E_SYNC and b + ngroups < B and b + ngroups != 40:
                assert st[b + ngroups] == oracle.TREE_E_SYNC, (b, st[b + ngroups])
        else:
            assert st[b] == oracle.TREE_OK, (b, st[b])
            np.testing.assert_array_equal(res["out_nodes"][b], ref["out_nodes"][b])
            np.testing.assert_array_equal(res["out_tokens"][b], ref["out_tokens"][b])
            assert res["out_count"][b] == ref["out_count"][b]
    say("  normal bound on the same buffers")
    dev.mask_build()
    dev.spec_accept()
    check_accept(dev.accept_results(), ref, "after give-up")
