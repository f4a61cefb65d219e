"""Edge cases across the entry points, on the GPU, against the oracle.

* an empty batch (B = 0) through every entry point: nothing is launched and
  every call returns OK;
* the largest trees the library takes (T_max = 256: four ancestor words per
  row) through mask, attention (one and several key ranges) and accept;
* one-position trees (the root alone) with an empty and a long prefix.
"""
import os

import numpy as np
import pytest

import oracle
from gpu_util import check_accept, check_attention, check_path_valid, need_gpu, say, sv_problem
from synth import make_instance

pytestmark = pytest.mark.gpu


def test_empty_batch_every_entry_point():
    need_gpu()
    import torch
    import eagle_tree_verification_attn_amd as sv
    say("edge: B = 0 through every entry point")
    i32 = dict(dtype=torch.int32, device="cuda")
    e = torch.empty((0,), **i32)
    T, Hq, Hkv, D, V = 5, 8, 2, 128, 64
    bf = dict(dtype=torch.bfloat16, device="cuda")
    q = torch.empty((0, T, Hq, D), **bf)
    kn = torch.empty((0, T, Hkv, D), **bf)
    kc = torch.empty((0, Hkv, 16, D), **bf)
    tree = sv.make_tree(torch.empty((0, T), **i32), e, torch.empty((0, T), **i32))
    anc = torch.empty((0, T, 1), dtype=torch.int64, device="cuda")
    depth = torch.empty((0, T), **i32)
    out = torch.empty_like(q)
    attn = sv.make_attn_args(q, kn, kn, kc, kc, e, out)
    f32 = dict(dtype=torch.float32, device="cuda")
    acc = sv.make_accept_args(torch.empty((0, T, V), **bf), torch.empty((0, T, V), **f32), torch.empty((0,), **f32),
                              torch.empty((0, T), **f32), torch.empty((0, T), **f32), torch.empty((0, T), **i32),
                              torch.empty((0, T), **i32), e, e)
    ws = torch.empty((256,), dtype=torch.uint8, device="cuda")
    assert sv.sv_tree_mask_build(tree, anc, depth, e) == sv.SV_OK
    assert sv.sv_tree_attn(tree, anc, e, attn, ws) == sv.SV_OK
    assert sv.sv_spec_accept(tree, e, acc, ws) == sv.SV_OK
    assert sv.sv_verify_step(tree, attn, acc, anc, depth, e, ws) == sv.SV_OK
    com = sv.make_commit_args(kn, kn, kc, kc, e, torch.empty((0,), **i32))
    assert sv.sv_commit_accepted(tree, e, torch.empty((0, T), **i32), e, com) == sv.SV_OK
    cfg = sv.SvEagle2Cfg(0, V, 2, 2, 3)
    assert sv.sv_eagle2_begin(cfg, None, e) == sv.SV_OK
    assert sv.sv_eagle2_expand(cfg, None, 0, torch.empty((0, 2, V), **f32)) == sv.SV_OK
    assert sv.sv_eagle2_finish(cfg, None, e, e, e, e, e) == sv.SV_OK
    torch.cuda.synchronize()


def _spec(**kw):
    s = dict(cfg_id=950, B=2, Hq=16, Hkv=2, D=128, dtype="bf16", logit_dtype="bf16", prefix_len=[300, 37],
             tree=("dynamic", 6, 12, 12, 48, 200, 255), T_max=256, V=3000, tau=[0.0, 0.9], sigma=1.0,
             draft_std=1.0, sibling_mode="wor")
    s.update(kw)
    return s


@pytest.mark.parametrize("lsplit", ["1", "3"])
def test_largest_trees_attention(lsplit):
    need_gpu()
    inst = make_instance(_spec(), 0, with_accept=False)
    assert inst.T_max == 256 and int(inst.num_nodes.max()) >= 200
    say(f"edge: T_max = 256 attention lsplit={lsplit} nodes={inst.num_nodes.tolist()}")
    old = os.environ.get("SV_ATTN_LSPLIT")
    os.environ["SV_ATTN_LSPLIT"] = lsplit
    try:
        dev = sv_problem(inst, with_accept=False)
        nbytes = dev.ws.numel()
        import eagle_tree_verification_attn_amd as sv
        need = sv.sv_workspace_bytes(dev.tree, dev.attn, None)
        if need > nbytes:
            import torch
            dev.ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
        dev.mask_build()
        dev.tree_attn()
        got = dev.attn_result()
    finally:
        if old is None:
            os.environ.pop("SV_ATTN_LSPLIT", None)
        else:
            os.environ["SV_ATTN_LSPLIT"] = old
    anc, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    assert (status == 0).all()
    ref = oracle.tree_attention(inst.q, inst.k_new, inst.v_new, inst.k_cache, inst.v_cache, inst.prefix_len, anc,
                                inst.num_nodes, status, inst.dtype)
    check_attention(got, ref, inst.dtype, label="T_max=256")


def test_largest_trees_accept():
    need_gpu()
    inst = make_instance(_spec(cfg_id=951, tau=[0.0, 0.9, 1.0, 0.0], B=4), 0, with_attn=False)
    say(f"edge: T_max = 256 accept nodes={inst.num_nodes.tolist()}")
    dev = sv_problem(inst, with_attn=False)
    dev.mask_build()
    dev.spec_accept()
    res = dev.accept_results()
    _, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    ref = oracle.spec_accept(inst.parent, inst.num_nodes, inst.tokens, inst.target_logits, inst.logit_dtype,
                             inst.q_probs, inst.temperature, inst.u_accept, inst.u_sample, status,
                             oracle.SIB_WITHOUT_REPLACEMENT)
    check_accept(res, ref, "T_max=256")
    for b in range(inst.B):
        if res["out_count"][b] > 0:
            check_path_valid(res, inst, b)


def test_root_only_trees_through_verification():
    need_gpu()
    spec = dict(cfg_id=952, B=3, Hq=8, Hkv=2, D=64, dtype="bf16", logit_dtype="bf16", prefix_len=[0, 1, 4000],
                tree=("chain", 0), V=2000, tau=[0.0, 1.0, 0.8], sigma=1.0, draft_std=2.0, sibling_mode="wor")
    inst = make_instance(spec, 0)
    assert inst.T_max == 1
    say("edge: root-only trees")
    dev = sv_problem(inst)
    dev.verify_step()
    ref = oracle.verify_step(inst)
    check_attention(dev.attn_result(), ref["attn"], "bf16", label="root only")
    res = dev.accept_results()
    check_accept(res, ref["accept"], "root only")
    assert res["out_count"].tolist() == [1, 1, 1]        # the bonus token alone


def test_no_prefix_at_all():
    """Every prefix empty (L_max = 0, no cache tensors): attention over the tree
    only, and the walk, against the oracle."""
    need_gpu()
    spec = dict(cfg_id=953, B=3, Hq=8, Hkv=2, D=128, dtype="bf16", logit_dtype="bf16", prefix_len=[0, 0, 0],
                tree=("dynamic", 1, 4, 1, 5, 1, 20), V=1500, tau=[0.0, 0.8, 1.0], sigma=1.0, draft_std=2.0,
                sibling_mode="wor", L_max=0)
    inst = make_instance(spec, 0)
    assert inst.L_max == 0
    say("edge: L_max = 0")
    dev = sv_problem(inst)
    dev.verify_step()
    ref = oracle.verify_step(inst)
    check_attention(dev.attn_result(), ref["attn"], "bf16", label="no prefix")
    check_accept(dev.accept_results(), ref["accept"], "no prefix")
