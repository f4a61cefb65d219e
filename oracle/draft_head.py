"""CPU oracle for the two-stage draft LM head (test infrastructure only).

Like the rest of this package, this is the plain definition the GPU kernels
are checked against; nothing on the product path imports it, and it shares no
code with the HIP library.

Source: [EAGLE-4 blog] (qingkeai.online, a former EAGLE Team member's post on
EAGLE-4), sections "EAGLE Efficient LM Head" (stage one picks candidates with
a cheap head, stage two recomputes their logits with the full head), "A
training-free version: Freq-aware SVD" and "A variant based on Local Top-k":

* low-rank factors: with token-frequency weights F = diag(f) (smoothed so
  f_i > 0), take the SVD F^(1/2) W = U S V^T, keep the top r singular
  triplets, and set A = F^(-1/2) U_r S_r, B = V_r^T (the page's formula);
* stage 1: u = B h;
* stage 2: approximate scores A u, but instead of writing all of them and
  taking a global top-k, each tile of the (shuffled) vocabulary keeps its own
  few best candidates (the page's conceptual pseudocode: one program per
  vocabulary tile, scores stay on chip, local top-k ids are stored);
* stage 3: exact logits W[ids] h for the candidates only.

Readings where the page is silent (listed in the design notes):

* the vocabulary shuffle is a fixed permutation ``perm`` applied offline: A's
  rows are stored in shuffled order, tiles are contiguous runs of ``tile``
  shuffled rows, and a candidate's token id is perm[position];
* precision: h, A, B and W are bf16; u is accumulated in float32 and stored as
  bf16 (the stage-2 operand); scores are float32 sums of bf16 products; each
  tile keeps its ``k_tile`` largest scores, ties to the lower shuffled
  position; candidates are ordered by tile, then by rank within the tile;
  exact logits are float32 sums of bf16 products (the oracle sums in float64);
* a last tile shorter than ``tile`` keeps min(k_tile, its length) candidates,
  and the rest of its slots are -1 with logit 0.

Pinned by ``tests/test_oracle_draft_head.py``: the weighted Eckart-Young
error of the factors (closed form), the plain truncated SVD when all weights
are equal, exact reconstruction at full rank, one tile equal to a brute-force
global top-k, every position's global best token among its candidates (the
best score is its tile's best), exact factors (r = d) giving candidate logits
equal to their scores, shuffle invariance of the single-tile result, and the
short last tile.
"""
import numpy as np


def bf16_round(x):
    """Round float64/float32 values to the nearest bfloat16 (ties to even),
    returned as float64."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def lowrank_factors(W, freq, r):
    """Frequency-weighted rank-r factors of W (n x d): A (n x r), B (r x d)
    with A B the best rank-r approximation of W in the norm weighted by F."""
    W = np.asarray(W, dtype=np.float64)
    f = np.asarray(freq, dtype=np.float64)
    assert (f > 0).all()
    s = np.sqrt(f)[:, None]
    U, S, Vt = np.linalg.svd(s * W, full_matrices=False)
    A = (U[:, :r] * S[:r]) / s
    B = Vt[:r]
    return A, B


def stage1(h, B):
    """u = B h for every position: h [N][d], B [r][d] -> u [N][r], stored as
    bf16 (values returned as float64)."""
    return bf16_round(np.asarray(h, dtype=np.float64) @ np.asarray(B, dtype=np.float64).T)


def stage2(u, A_sh, tile, k_tile):
    """Scores of every shuffled vocabulary row and each tile's k_tile best per
    position.  u [N][r], A_sh [n][r] (rows in shuffled order).  Returns
    (scores [N][n], cand_pos [N][n_tiles * k_tile] shuffled positions, -1
    padded, margins [N][n_tiles]: for each tile the gap between its k_tile-th
    and next score, inf when the tile has no next)."""
    u = np.asarray(u, dtype=np.float64)
    A = np.asarray(A_sh, dtype=np.float64)
    N = u.shape[0]
    n = A.shape[0]
    scores = u @ A.T
    n_tiles = (n + tile - 1) // tile
    cand = np.full((N, n_tiles * k_tile), -1, dtype=np.int64)
    margins = np.full((N, n_tiles), np.inf)
    for t in range(n_tiles):
        lo, hi = t * tile, min(n, (t + 1) * tile)
        kk = min(k_tile, hi - lo)
        for i in range(N):
            seg = scores[i, lo:hi]
            order = np.lexsort((np.arange(hi - lo), -seg))   # score descending, then position
            cand[i, t * k_tile:t * k_tile + kk] = lo + order[:kk]
            if hi - lo > kk:
                margins[i, t] = seg[order[kk - 1]] - seg[order[kk]]
    return scores, cand, margins


def stage3(h, W, perm, cand_pos):
    """Exact logits of the candidates: W[perm[pos]] . h (float64 sums of the
    stored values); -1 slots give id -1 and logit 0."""
    h = np.asarray(h, dtype=np.float64)
    perm = np.asarray(perm)
    ids = np.where(cand_pos >= 0, perm[np.maximum(cand_pos, 0)], -1)
    logits = np.zeros(cand_pos.shape, dtype=np.float64)
    for i in range(cand_pos.shape[0]):
        ok = ids[i] >= 0
        logits[i, ok] = np.asarray(W[ids[i, ok]], dtype=np.float64) @ h[i]   # only the gathered rows
    return ids, logits


def two_stage_head(h, A_sh, B, perm, W, tile, k_tile):
    """The whole head: returns dict(u, scores, cand_pos, cand_ids, cand_logits, margins)."""
    u = stage1(h, B)
    scores, cand_pos, margins = stage2(u, A_sh, tile, k_tile)
    ids, logits = stage3(h, W, perm, cand_pos)
    return dict(u=u, scores=scores, cand_pos=cand_pos, cand_ids=ids, cand_logits=logits, margins=margins)
