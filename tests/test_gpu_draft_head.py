"""GPU two-stage draft LM head (sv_draft_head) against the oracle.

* u = B h is bit-exact when the inputs make float32 sums exact (values in
  multiples of 1/8), and within one bf16 step otherwise;
* the candidate ids of every (position, tile) are bit-exact, except tiles
  whose oracle gap between the k_tile-th and the next score is within the
  float32 rounding bound of the scores (then both selections must still be
  k_tile rows of that tile);
* the exact logits are within the float32 summation bound d * 2^-24 * sum|w h|.

Cases: several tile sizes and k_tile, position counts that do and do not fill
a 16-wide MFMA tile, vocabularies with a short last tile, k_tile above a short
tile's length, Gaussian inputs, and a single-sequence drafter step at full
size (8 positions, d = 8192, r = 256, V = 128256).
"""
import numpy as np
import pytest

from oracle import draft_head as dh
from gpu_util import need_gpu, say
from synth import f32_from_bf16_bits, make_head_inputs

pytestmark = pytest.mark.gpu


def _to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run_gpu(inp, tile, k_tile, W_dev=None):
    import torch
    import eagle_tree_verification_attn_amd as sv
    N, d = inp["h"].shape
    r, n = inp["B"].shape[0], inp["A_sh"].shape[0]
    C = -(-n // tile) * k_tile
    h, B, A = _to_dev(inp["h"]), _to_dev(inp["B"]), _to_dev(inp["A_sh"])
    W = W_dev if W_dev is not None else _to_dev(inp["W"])
    perm = torch.from_numpy(inp["perm"]).cuda()
    u = torch.full((N, r), 7.0, dtype=torch.bfloat16, device="cuda")
    ids = torch.full((N, C), -7, dtype=torch.int32, device="cuda")
    logits = torch.full((N, C), 7.0, dtype=torch.float32, device="cuda")
    args = sv.make_head_args(h, B, A, perm, W, u, ids, logits, tile, k_tile)
    sv.sv_draft_head(args)
    torch.cuda.synchronize()
    return dict(u=u.float().cpu().numpy().astype(np.float64), ids=ids.cpu().numpy(), logits=logits.cpu().numpy())


def _check(got, ref, h, W, n, tile, k_tile, exact_u, label):
    if exact_u:
        np.testing.assert_array_equal(got["u"], ref["u"], err_msg=f"{label} u")
    else:
        ulp = np.abs(ref["u"]) * 2.0 ** -7 + 1e-30
        assert (np.abs(got["u"] - ref["u"]) <= ulp).all(), label
    N = got["ids"].shape[0]
    n_tiles = -(-n // tile)
    scale = np.abs(ref["scores"]).max()
    tol = 1e-5 * scale
    exempt = 0
    for i in range(N):
        for t in range(n_tiles):
            g = got["ids"][i, t * k_tile:(t + 1) * k_tile]
            e = ref["cand_ids"][i, t * k_tile:(t + 1) * k_tile]
            if ref["margins"][i, t] > tol:
                assert g.tolist() == e.tolist(), (label, i, t, g, e)
            else:
                exempt += 1
                assert (g >= 0).sum() == (e >= 0).sum()
    # exact logits of the GPU's own candidates, float64 reference
    ok = got["ids"] >= 0
    for i in range(N):
        rows = W[got["ids"][i][ok[i]]]
        ref_l = rows @ h[i]
        bound = h.shape[1] * 2.0 ** -24 * (np.abs(rows) @ np.abs(h[i])) + 1e-30
        assert (np.abs(got["logits"][i][ok[i]] - ref_l) <= bound).all(), (label, i)
        assert (got["logits"][i][~ok[i]] == 0).all()
    return exempt


CASES = [
    # N, d, r, n, tile, k_tile, quantized
    (5, 256, 64, 1000, 64, 3, True),
    (19, 512, 96, 3001, 256, 8, True),       # two position tiles, short last vocabulary tile
    (8, 256, 32, 2000, 16, 1, True),         # smallest tiles
    (3, 128, 64, 1030, 128, 8, True),        # last tile of 6 rows < k_tile
    (16, 1024, 128, 5000, 256, 2, False),    # Gaussian inputs
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}_d{c[1]}_r{c[2]}_n{c[3]}_t{c[4]}_k{c[5]}{'' if c[6] else '_gauss'}"
                                             for c in CASES])
def test_draft_head_matches_oracle(case):
    need_gpu()
    N, d, r, n, tile, k_tile, quant = case
    inp = make_head_inputs(N, d, r, n, seed=sum(case[:6]), quantized=quant)
    say(f"draft head N={N} d={d} r={r} n={n} tile={tile} k_tile={k_tile} quantized={quant}")
    got = _run_gpu(inp, tile, k_tile)
    f = {k: f32_from_bf16_bits(inp[k]).astype(np.float64) for k in ("h", "B", "A_sh", "W")}
    ref = dh.two_stage_head(f["h"], f["A_sh"], f["B"], inp["perm"], f["W"], tile, k_tile)
    _check(got, ref, f["h"], f["W"], n, tile, k_tile, quant, str(case))


def test_draft_head_full_size_drafter_step():
    """8 positions (one sequence's frontier), d = 8192, r = 256, V = 128256,
    tiles of 256 with 2 candidates each; W is made on the device (seeded torch
    generator, values in multiples of 1/8) and the oracle reads the rows it
    needs from it."""
    need_gpu()
    import torch
    N, d, r, n, tile, k_tile = 8, 8192, 256, 128256, 256, 2
    inp = make_head_inputs(N, d, r, n, seed=1, quantized=True, with_W=False)
    g = torch.Generator(device="cuda").manual_seed(11)
    W_dev = (torch.randint(-8, 9, (n, d), generator=g, device="cuda", dtype=torch.int32).float() / 8.0).to(torch.bfloat16)
    say("draft head full size: N=8 d=8192 r=256 n=128256 tile=256 k_tile=2")
    got = _run_gpu(inp, tile, k_tile, W_dev=W_dev)
    f = {k: f32_from_bf16_bits(inp[k]).astype(np.float64) for k in ("h", "B", "A_sh")}
    u = dh.stage1(f["h"], f["B"])
    scores, cand_pos, margins = dh.stage2(u, f["A_sh"], tile, k_tile)
    ids_needed = np.unique(np.concatenate([inp["perm"][cand_pos[cand_pos >= 0]], got["ids"][got["ids"] >= 0]]))
    W_host = np.zeros((n, d), dtype=np.float32)
    W_host[ids_needed] = W_dev[torch.from_numpy(ids_needed).cuda()].float().cpu().numpy()
    ids, logits = dh.stage3(f["h"], W_host, inp["perm"], cand_pos)
    ref = dict(u=u, scores=scores, cand_pos=cand_pos, cand_ids=ids, cand_logits=logits, margins=margins)
    exempt = _check(got, ref, f["h"], W_host, n, tile, k_tile, True, "full size")
    assert exempt < 0.01 * N * (-(-n // tile))
    # every position's best approximate score is among its candidates
    for i in range(N):
        assert inp["perm"][int(np.argmax(scores[i]))] in got["ids"][i].tolist()
