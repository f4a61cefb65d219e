"""Pins for the oracle's two-stage draft LM head (CPU only).

* factors: the F-weighted error of the rank-r factors equals the sum of the
  discarded squared singular values of F^(1/2) W (Eckart-Young, closed form);
  with equal weights they reproduce numpy's plain truncated SVD; at full rank
  A B = W exactly;
* local top-k: with one tile it equals a brute-force global top-k; with many
  tiles, every position's best-scoring token is among its candidates; the
  candidates of each tile are that tile's best by brute force;
* exact stage: with exact factors (A = W, B = identity) the candidate logits
  equal their stage-two scores;
* the shuffle: with one tile the candidate token set does not depend on it;
* a short last tile keeps fewer candidates and pads with -1;
* bf16 rounding: ties go to even, and values already in bf16 are unchanged.
"""
import numpy as np
import pytest

from oracle import draft_head as dh


def _bf16(rng, shape, scale=1.0):
    return dh.bf16_round(rng.normal(0, scale, shape))


def test_bf16_rounding():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9])
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even (1); 1 + 3 * 2^-8 -> 1 + 2^-6
    np.testing.assert_array_equal(dh.bf16_round(x), [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0])
    y = dh.bf16_round(np.random.default_rng(0).normal(size=100))
    np.testing.assert_array_equal(dh.bf16_round(y), y)


@pytest.mark.parametrize("r", [1, 3, 7])
def test_factors_weighted_error_is_the_discarded_spectrum(r):
    rng = np.random.default_rng(r)
    W = rng.normal(size=(40, 12))
    f = rng.uniform(0.1, 5.0, 40)
    A, B = dh.lowrank_factors(W, f, r)
    err = np.sum(f[:, None] * (W - A @ B) ** 2)
    s = np.linalg.svd(np.sqrt(f)[:, None] * W, compute_uv=False)
    assert abs(err - np.sum(s[r:] ** 2)) <= 1e-9 * np.sum(s ** 2)


def test_factors_equal_weights_is_plain_truncated_svd():
    rng = np.random.default_rng(5)
    W = rng.normal(size=(30, 10))
    A, B = dh.lowrank_factors(W, np.ones(30) * 3.0, 4)
    U, S, Vt = np.linalg.svd(W, full_matrices=False)
    np.testing.assert_allclose(A @ B, (U[:, :4] * S[:4]) @ Vt[:4], atol=1e-10)


def test_factors_full_rank_reconstruct():
    rng = np.random.default_rng(6)
    W = rng.normal(size=(20, 8))
    A, B = dh.lowrank_factors(W, rng.uniform(0.5, 2, 20), 8)
    np.testing.assert_allclose(A @ B, W, atol=1e-10)


def _problem(seed, N=3, d=24, r=6, n=50):
    rng = np.random.default_rng(seed)
    h = _bf16(rng, (N, d))
    W = _bf16(rng, (n, d), 0.2)
    A, B = dh.lowrank_factors(W, rng.uniform(0.5, 2.0, n), r)
    perm = rng.permutation(n)
    return h, dh.bf16_round(A[perm]), dh.bf16_round(B), perm, W


@pytest.mark.parametrize("k", [1, 3, 5])
def test_one_tile_is_global_top_k(k):
    h, A_sh, B, perm, W = _problem(1)
    out = dh.two_stage_head(h, A_sh, B, perm, W, tile=len(perm), k_tile=k)
    for i in range(h.shape[0]):
        brute = np.argsort(-out["scores"][i], kind="stable")[:k]
        assert out["cand_pos"][i].tolist() == brute.tolist()


@pytest.mark.parametrize("tile,k", [(7, 1), (10, 2), (16, 3)])
def test_tiles_keep_their_best_and_the_global_best(tile, k):
    h, A_sh, B, perm, W = _problem(2)
    out = dh.two_stage_head(h, A_sh, B, perm, W, tile=tile, k_tile=k)
    n = len(perm)
    for i in range(h.shape[0]):
        sc = out["scores"][i]
        assert int(np.argmax(sc)) in out["cand_pos"][i].tolist()
        assert perm[int(np.argmax(sc))] in out["cand_ids"][i].tolist()
        for t in range((n + tile - 1) // tile):
            lo, hi = t * tile, min(n, (t + 1) * tile)
            got = out["cand_pos"][i][t * k:(t + 1) * k]
            got = got[got >= 0]
            best = set((lo + np.argsort(-sc[lo:hi], kind="stable")[:min(k, hi - lo)]).tolist())
            assert set(got.tolist()) == best


def test_exact_factors_give_logits_equal_to_scores():
    rng = np.random.default_rng(3)
    N, d, n = 2, 16, 30
    h = _bf16(rng, (N, d))
    W = _bf16(rng, (n, d), 0.3)
    perm = rng.permutation(n)
    # A = W (shuffled), B = identity: stage 1 returns h rounded to bf16 = h
    out = dh.two_stage_head(h, W[perm], np.eye(d), perm, W, tile=8, k_tile=2)
    for i in range(N):
        ok = out["cand_pos"][i] >= 0
        np.testing.assert_allclose(out["cand_logits"][i][ok], out["scores"][i][out["cand_pos"][i][ok]], rtol=1e-12)


def test_single_tile_candidates_do_not_depend_on_the_shuffle():
    h, A_sh, B, perm, W = _problem(4)
    A = np.empty_like(A_sh)
    A[perm] = A_sh                      # back to token order
    a = dh.two_stage_head(h, A_sh, B, perm, W, tile=len(perm), k_tile=4)
    ident = np.arange(len(perm))
    b = dh.two_stage_head(h, A, B, ident, W, tile=len(perm), k_tile=4)
    for i in range(h.shape[0]):
        assert sorted(a["cand_ids"][i].tolist()) == sorted(b["cand_ids"][i].tolist())


def test_short_last_tile():
    h, A_sh, B, perm, W = _problem(5, n=23)
    out = dh.two_stage_head(h, A_sh, B, perm, W, tile=10, k_tile=4)     # tiles of 10, 10, 3
    assert out["cand_pos"].shape[1] == 12
    last = out["cand_pos"][:, 8:]
    assert (last[:, :3] >= 20).all() and (last[:, 3] == -1).all()
    assert (out["cand_ids"][:, 11] == -1).all() and (out["cand_logits"][:, 11] == 0).all()
    assert np.isinf(out["margins"][:, 2]).all()
