"""Pins for the oracle's tree mask and tree attention (CPU only).

Mask: the worked example tree printed on the speculative-decoding lesson page,
the recursive ancestor identity, popcount = depth + 1, the chain case reducing
to the causal triangle, and the validation statuses.

Attention: for every root-to-leaf path, tree attention at the path's nodes must
equal plain causal attention over [prefix; path], computed by a library routine
(torch's scaled_dot_product_attention on the CPU in float64, with its own GQA
head mapping).  The chain and the single-position case reduce to causal and
decode attention.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import bf16_bits_from_f32, tree_from_widths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- mask
def test_mask_lesson_example_tree():
    g = _golden("lesson_example_tree.json")
    parent = np.array([g["parent"]], dtype=np.int32)
    T = len(g["parent"])
    anc, bits, depth, status = oracle.tree_mask(parent, [T], T)
    assert status[0] == oracle.TREE_OK
    for i, want in enumerate(g["ancestor_or_self"]):
        assert sorted(np.nonzero(anc[0, i])[0].tolist()) == want
        assert int(bits[0, i, 0]) == sum(1 << j for j in want)
    assert depth[0].tolist() == g["depth"]
    # branches do not see each other
    assert not anc[0, 1, 2] and not anc[0, 3, 4] and not anc[0, 5, 3]


@pytest.mark.parametrize("seed", range(5))
def test_mask_recursive_identity_and_depth(seed):
    rng = np.random.default_rng(seed)
    widths = [int(w) for w in rng.integers(1, 9, size=int(rng.integers(1, 9)))]
    par = tree_from_widths(widths, rng)
    T = len(par)
    T_max = T + int(rng.integers(0, 70))
    parent = np.full((1, T_max), -1, dtype=np.int32)
    parent[0, :T] = par
    anc, bits, depth, status = oracle.tree_mask(parent, [T], T_max)
    assert status[0] == 0
    for i in range(1, T):
        want = anc[0, par[i]].copy()
        want[i] = True
        assert np.array_equal(anc[0, i], want)
    assert anc[0, 0].sum() == 1 and anc[0, 0, 0]
    assert np.array_equal(anc[0].sum(axis=1)[:T], depth[0, :T] + 1)
    # lower triangular, padding rows/cols empty
    assert not np.any(np.triu(anc[0], 1))
    assert not anc[0, T:].any() and not anc[0, :, T:].any()
    # packed bits agree with the boolean mask
    for i in range(T_max):
        for j in range(T_max):
            bit = (int(bits[0, i, j // 64]) >> (j % 64)) & 1
            assert bit == int(anc[0, i, j])


def test_mask_chain_is_causal_triangle():
    T = 70
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    anc, bits, depth, status = oracle.tree_mask(parent, [T], T)
    assert np.array_equal(anc[0], np.tril(np.ones((T, T), dtype=bool)))
    assert depth[0].tolist() == list(range(T))
    assert bits.shape[2] == 2


def test_mask_validation_statuses():
    T_max = 6
    parent = np.array([
        [-1, 0, 0, 1, 2, 3],     # ok
        [0, 0, 0, 1, 2, 3],      # root has a parent
        [-1, 0, 2, 1, 2, 3],     # parent[2] == 2 (not < i)
        [-1, 0, 0, 7, 2, 3],     # parent out of range
        [-1, 0, 0, 1, 2, 3],     # count 0
        [-1, 0, 0, 1, 2, 3],     # count > T_max
        [-1, -1, 0, 1, 2, 3],    # negative parent for a draft node
    ], dtype=np.int32)
    counts = [6, 6, 6, 6, 0, 7, 6]
    anc, bits, depth, status = oracle.tree_mask(parent, counts, T_max)
    assert status.tolist() == [0, oracle.TREE_E_ROOT, oracle.TREE_E_PARENT, oracle.TREE_E_PARENT,
                               oracle.TREE_E_COUNT, oracle.TREE_E_COUNT, oracle.TREE_E_PARENT]
    assert not anc[1:].any() and not depth[1:].any()
    # the padding beyond T_b is never checked
    p2 = np.array([[-1, 0, 99, 99]], dtype=np.int32)
    _, _, _, st = oracle.tree_mask(p2, [2], 4)
    assert st[0] == 0


# ----------------------------------------------------------------------------- attention
def _paths(parent, T):
    kids = {i: [] for i in range(T)}
    for i in range(1, T):
        kids[int(parent[i])].append(i)
    out = []

    def rec(n, acc):
        if not kids[n]:
            out.append(acc + [n])
        for c in kids[n]:
            rec(c, acc + [n])
    rec(0, [])
    return out


def _sdpa_path(qf, knf, vnf, kcf, vcf, b, L, path, scale):
    """Causal attention over [prefix; path] for the path's queries (float64)."""
    Qp = torch.from_numpy(qf[b, path]).transpose(0, 1)              # Hq x P x D
    Kp = torch.from_numpy(np.concatenate([kcf[b, :, :L], knf[b, path].transpose(1, 0, 2)], axis=1))
    Vp = torch.from_numpy(np.concatenate([vcf[b, :, :L], vnf[b, path].transpose(1, 0, 2)], axis=1))
    P = len(path)
    mask = torch.ones(P, L + P, dtype=torch.bool)
    mask[:, L:] = torch.tril(torch.ones(P, P, dtype=torch.bool))
    o = F.scaled_dot_product_attention(Qp[None], Kp[None], Vp[None], attn_mask=mask,
                                       scale=scale, enable_gqa=True)
    return o[0].transpose(0, 1).numpy()                              # P x Hq x D


def _rand_attn(rng, B, T_max, Hq, Hkv, D, L_max, dtype):
    def n(*shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return bf16_bits_from_f32(x) if dtype == "bf16" else x
    return (n(B, T_max, Hq, D), n(B, T_max, Hkv, D), n(B, T_max, Hkv, D),
            n(B, Hkv, L_max, D), n(B, Hkv, L_max, D))


@pytest.mark.parametrize("dtype,G,D,seed", [("f32", 1, 64, 0), ("bf16", 4, 128, 1),
                                            ("bf16", 8, 64, 2), ("f32", 5, 32, 3)])
def test_attention_equals_causal_attention_on_every_path(dtype, G, D, seed):
    rng = np.random.default_rng(seed)
    B, Hkv = 3, 2
    Hq = G * Hkv
    trees = [tree_from_widths([2, 3, 3], rng), tree_from_widths([1, 4, 2, 2], rng),
             np.array([-1], dtype=np.int32)]
    T_max = max(len(t) for t in trees) + 2
    parent = np.full((B, T_max), -1, dtype=np.int32)
    for b, t in enumerate(trees):
        parent[b, :len(t)] = t
    num = np.array([len(t) for t in trees], dtype=np.int32)
    prefix = np.array([37, 0, 65], dtype=np.int32)
    q, kn, vn, kc, vc = _rand_attn(rng, B, T_max, Hq, Hkv, D, 65, dtype)
    anc, _, _, status = oracle.tree_mask(parent, num, T_max)
    out = oracle.tree_attention(q, kn, vn, kc, vc, prefix, anc, num, status, dtype)
    qf, knf, vnf, kcf, vcf = (oracle.to_f64(a, dtype) for a in (q, kn, vn, kc, vc))
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        T = int(num[b])
        for path in _paths(parent[b], T):
            ref = _sdpa_path(qf, knf, vnf, kcf, vcf, b, int(prefix[b]), path, scale)
            np.testing.assert_allclose(out[b, path], ref, rtol=1e-12, atol=1e-12)
        assert not out[b, T:].any()


def test_attention_chain_equals_causal_and_explicit_scale():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, T, L = 2, 8, 2, 64, 9, 50
    parent = np.tile(np.arange(-1, T - 1, dtype=np.int32), (B, 1))
    num = np.array([T, T], dtype=np.int32)
    prefix = np.array([L, 11], dtype=np.int32)
    q, kn, vn, kc, vc = _rand_attn(rng, B, T, Hq, Hkv, D, L, "f32")
    anc, _, _, status = oracle.tree_mask(parent, num, T)
    scale = np.float32(0.3)
    out = oracle.tree_attention(q, kn, vn, kc, vc, prefix, anc, num, status, "f32", scale=scale)
    qf, knf, vnf, kcf, vcf = (oracle.to_f64(a, "f32") for a in (q, kn, vn, kc, vc))
    for b in range(B):
        ref = _sdpa_path(qf, knf, vnf, kcf, vcf, b, int(prefix[b]), list(range(T)), float(scale))
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_attention_invalid_tree_rows_are_zero():
    rng = np.random.default_rng(3)
    parent = np.array([[-1, 0, 0], [0, 0, 1]], dtype=np.int32)
    num = np.array([3, 3])
    q, kn, vn, kc, vc = _rand_attn(rng, 2, 3, 2, 1, 16, 4, "f32")
    anc, _, _, status = oracle.tree_mask(parent, num, 3)
    out = oracle.tree_attention(q, kn, vn, kc, vc, np.array([4, 4]), anc, num, status, "f32")
    assert status.tolist() == [0, oracle.TREE_E_ROOT]
    assert np.abs(out[0]).sum() > 0 and not out[1].any()


def test_to_f64_bf16_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    got = oracle.to_f64(bits, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
