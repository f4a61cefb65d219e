"""Pins for the oracle's commit of the accepted path (CPU only).

* path equivalence: after the commit, plain causal attention of every
  committed position's query over the extended cache reproduces that
  position's tree-attention output (float64, library attention), so the rows,
  their order and the KV-head mapping are fixed by the tree-attention
  definition rather than restated;
* features cross-check: features taken from the K rows of one head come out
  equal to the rows the commit wrote into that head's cache;
* special cases: a cache without room, an invalid sequence, the root alone,
  path entries out of range.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import make_instance


def _spec(**kw):
    s = dict(cfg_id=500, B=5, Hq=6, Hkv=2, D=32, dtype="f32", logit_dtype="f32", prefix_len=[9, 0, 23, 4, 15],
             tree=("dynamic", 1, 5, 1, 4, 1, 20), V=40, tau=("choice", [0.0, 0.7, 1.0]), sigma=0.5,
             draft_std=1.0, sibling_mode="wor")
    s.update(kw)
    return s


def _verify(inst):
    anc, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    att = oracle.tree_attention(inst.q, inst.k_new, inst.v_new, inst.k_cache, inst.v_cache,
                                inst.prefix_len, anc, inst.num_nodes, status, inst.dtype)
    acc = oracle.spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits,
                             inst.logit_dtype, inst.q_probs, inst.temperature, inst.u_accept,
                             inst.u_sample, status)
    return status, att, acc


@pytest.mark.parametrize("seed", range(4))
def test_commit_then_causal_attention_reproduces_tree_attention(seed):
    inst = make_instance(_spec(L_max=23 + 22), seed)
    status, att, acc = _verify(inst)
    com = oracle.commit_accepted(inst.k_new, inst.v_new, inst.k_cache, inst.v_cache, inst.prefix_len,
                                 inst.num_nodes, acc["status"], acc["out_nodes"], acc["out_count"])
    G = inst.Hq // inst.Hkv
    scale = 1.0 / math.sqrt(inst.D)
    checked = 0
    for b in range(inst.B):
        if acc["status"][b] != oracle.TREE_OK:
            continue
        c = int(acc["out_count"][b])
        L = int(inst.prefix_len[b])
        assert com["prefix_len"][b] == L + c
        positions = [0] + [int(n) for n in acc["out_nodes"][b][:c - 1]]
        kc = torch.from_numpy(oracle.to_f64(com["k_cache"][b], inst.dtype))      # Hkv x L_max x D
        vc = torch.from_numpy(oracle.to_f64(com["v_cache"][b], inst.dtype))
        for j, n in enumerate(positions):
            q = torch.from_numpy(oracle.to_f64(inst.q[b, n], inst.dtype))        # Hq x D
            keys = L + j + 1                                                     # prefix + committed 0..j
            o = F.scaled_dot_product_attention(q[:, None, :], kc.repeat_interleave(G, 0)[:, :keys],
                                               vc.repeat_interleave(G, 0)[:, :keys], scale=scale)
            np.testing.assert_allclose(o[:, 0].numpy(), att[b, n], rtol=1e-12, atol=1e-12)
            checked += 1
        # rows outside [L, L + c) are untouched
        np.testing.assert_array_equal(com["k_cache"][b][:, :L], inst.k_cache[b][:, :L])
        np.testing.assert_array_equal(com["v_cache"][b][:, L + c:], inst.v_cache[b][:, L + c:])
    assert checked > 0


def test_commit_features_match_committed_cache_rows():
    inst = make_instance(_spec(L_max=50, dtype="bf16"), 7)
    _, _, acc = _verify(inst)
    h = 1
    feat_in = np.ascontiguousarray(inst.k_new[:, :, h, :])                      # F = D rows of head h
    com = oracle.commit_accepted(inst.k_new, inst.v_new, inst.k_cache, inst.v_cache, inst.prefix_len,
                                 inst.num_nodes, acc["status"], acc["out_nodes"], acc["out_count"], feat_in)
    for b in range(inst.B):
        if acc["status"][b] != oracle.TREE_OK:
            continue
        c, L = int(acc["out_count"][b]), int(inst.prefix_len[b])
        np.testing.assert_array_equal(com["feat_out"][b, :c], com["k_cache"][b, h, L:L + c])
        assert not com["feat_out"][b, c:].any()


def test_commit_special_cases():
    inst = make_instance(_spec(B=5, prefix_len=[10, 3, 6, 2, 2], L_max=12, tree=("widths", [2, 2])), 3)
    status, _, acc = _verify(inst)
    nodes = acc["out_nodes"].copy()
    count = acc["out_count"].copy()
    st = acc["status"].copy()
    st[:] = oracle.TREE_OK
    count[0] = 3                  # 10 + 3 > 12: no room
    count[1] = 1                  # the root alone
    nodes[1, :] = -1
    st[2] = oracle.TREE_E_PARENT  # invalid sequence: left alone
    count[3], nodes[3, 0] = 2, 5  # a path entry outside [1, T_b) (T_b = 5)
    count[4] = 6                  # more than T_b positions
    com = oracle.commit_accepted(inst.k_new, inst.v_new, inst.k_cache, inst.v_cache, inst.prefix_len,
                                 inst.num_nodes, st, nodes, count)
    assert com["status"].tolist() == [oracle.TREE_E_CACHE, oracle.TREE_OK, oracle.TREE_E_PARENT,
                                      oracle.TREE_E_PATH, oracle.TREE_E_PATH]
    assert com["prefix_len"].tolist() == [10, 4, 6, 2, 2]
    np.testing.assert_array_equal(com["k_cache"][0], inst.k_cache[0])
    np.testing.assert_array_equal(com["k_cache"][2], inst.k_cache[2])
    np.testing.assert_array_equal(com["k_cache"][1][:, 3], inst.k_new[1, 0])
    np.testing.assert_array_equal(com["v_cache"][1][:, 3], inst.v_new[1, 0])
