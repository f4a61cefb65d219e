"""Helpers for the GPU parity tests: device checks and comparisons with the oracle."""
import os
import sys

import numpy as np
import pytest

import oracle

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL, F32_RTOL = 1e-5, 1e-5
# Per output row (sequence, position, head: D values), bf16: |got - ref|_2 <=
# BF16_ROW_RTOL |ref|_2.  The kernel's own rounding gives about 0.1% rms from
# the bf16 output and 0.1% from the bf16 weights of P; a key left out of or
# wrongly added to the softmax moves a row by its weight, which the
# element-wise bound alone misses where long prefixes make outputs small.
BF16_ROW_RTOL = 1e-2


def have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def need_gpu():
    if not have_gpu():
        pytest.skip("no GPU on this host")


def say(msg):
    """Progress line naming the case (flushed before each GPU step)."""
    print(msg, flush=True)
    sys.stdout.flush()


def sv_problem(inst, **kw):
    from eagle_tree_verification_attn_amd.problem import DeviceProblem
    return DeviceProblem(inst, **kw)


def check_mask(dev, inst):
    import torch
    torch.cuda.synchronize()
    anc, depth, status = dev.mask_results()
    _, ref_bits, ref_depth, ref_status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    np.testing.assert_array_equal(status, ref_status)
    np.testing.assert_array_equal(anc, ref_bits)
    np.testing.assert_array_equal(depth, ref_depth)
    return ref_status


def check_attention(got, ref, dtype, rows=None, label=""):
    """Element-wise comparison at the stated tolerance; rows = list of (b, h)."""
    atol, rtol = (BF16_ATOL, BF16_RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)
    if rows is None:
        g, r = got, ref
    else:
        g = np.stack([got[b, :, h] for b, h in rows])
        r = np.stack([ref[b, :, h] for b, h in rows])
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{label}: {bad.sum()} of {bad.size} outside tolerance; max err "
                             f"{err.max():.3e}; first {idx.tolist()}")
    if dtype == "bf16":
        rn = np.sqrt((r * r).sum(axis=-1))
        en = np.sqrt(((g - r) ** 2).sum(axis=-1))
        live = rn > 0
        rel = np.where(live, en / np.where(live, rn, 1.0), 0.0)
        if (rel > BF16_ROW_RTOL).any():
            idx = np.argwhere(rel > BF16_ROW_RTOL)[:5]
            raise AssertionError(f"{label}: {(rel > BF16_ROW_RTOL).sum()} rows with relative L2 error above "
                                 f"{BF16_ROW_RTOL}; max {rel.max():.3e}; first {idx.tolist()}")
        say(f"{label}: max abs err {err.max():.3e}, max row rel L2 err {rel.max():.3e}")
    return float(err.max())


def check_accept(res, ref, label=""):
    """GPU accept outputs vs oracle: bit-exact up to the first decision whose
    oracle margin is below the exemption threshold; after it, a valid path."""
    B = len(ref["out_count"])
    exempt = 0
    for b in range(B):
        assert res["status"][b] == ref["status"][b], (label, b, res["status"][b], ref["status"][b])
        w = ref["walks"][b]
        if w is None:
            assert res["out_count"][b] == 0 and (res["out_nodes"][b] == -1).all() \
                and (res["out_tokens"][b] == -1).all(), (label, b)
            continue
        if w["exempt_at"] is None:
            np.testing.assert_array_equal(res["out_nodes"][b], ref["out_nodes"][b], err_msg=f"{label} b={b} nodes")
            np.testing.assert_array_equal(res["out_tokens"][b], ref["out_tokens"][b], err_msg=f"{label} b={b} tokens")
            assert res["out_count"][b] == ref["out_count"][b], (label, b)
            assert res["out_passes"][b] == w["passes"], (label, b, res["out_passes"][b], w["passes"])
        else:
            exempt += 1
            k = w["exempt_at"]
            np.testing.assert_array_equal(res["out_nodes"][b][:k], ref["out_nodes"][b][:k])
            assert res["out_count"][b] >= k + 1
    return exempt


def check_path_valid(res, inst, b):
    """The GPU's accepted path is a root-descending chain with matching tokens."""
    n = 0
    cnt = int(res["out_count"][b])
    for i in range(cnt - 1):
        c = int(res["out_nodes"][b][i])
        assert int(inst.parent[b][c]) == n
        assert int(res["out_tokens"][b][i]) == int(inst.tokens[b][c])
        n = c
    assert 0 <= int(res["out_tokens"][b][cnt - 1]) < inst.V
