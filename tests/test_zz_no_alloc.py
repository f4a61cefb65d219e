"""sv_verify_step_noalloc (the step with the library's own scratch memory)
against sv_verify_step with a caller workspace: the same results, bit for
bit, on two calls in a row (the second with a smaller problem, so it finds
the first call's contents in the scratch array), and a host-side rejection of
a problem that needs more scratch than the library holds."""
import ctypes
import os

import numpy as np
import pytest

import eagle_tree_verification_attn_amd as sv

SCRATCH_BYTES = 64 << 20


def test_noalloc_rejects_oversized_problem_on_the_host():
    """No GPU needed: the size check comes before any launch (the pointers
    below are never dereferenced)."""
    fake = 0x10000
    B, T, Hq, Hkv, D, L = 8, 65, 64, 8, 128, 2048
    tree = sv.SvTree(B, T, ctypes.c_void_p(fake), ctypes.c_void_p(fake), ctypes.c_void_p(fake))
    attn = sv.SvAttnArgs(Hq, Hkv, D, L, sv.SV_BF16, 0.0, fake, fake, fake, fake, fake, fake, fake)
    acc = sv.SvAcceptArgs(128256, sv.SV_BF16, 0, fake, fake, fake, fake, fake, fake, fake, fake, None)
    old = os.environ.get("SV_ATTN_LSPLIT")
    os.environ["SV_ATTN_LSPLIT"] = "16"     # partial results: 8*65*64*16*128*4 bytes = 272 MB
    try:
        need = sv.lib().sv_workspace_bytes(ctypes.byref(tree), ctypes.byref(attn), ctypes.byref(acc))
        assert need > SCRATCH_BYTES
        rc = sv.lib().sv_verify_step_noalloc(ctypes.byref(tree), ctypes.byref(attn), ctypes.byref(acc),
                                             ctypes.c_void_p(fake), ctypes.c_void_p(fake), ctypes.c_void_p(fake), None)
    finally:
        if old is None:
            os.environ.pop("SV_ATTN_LSPLIT", None)
        else:
            os.environ["SV_ATTN_LSPLIT"] = old
    assert rc == sv.SV_E_WORKSPACE
    assert b"more than the 67108864" in sv.lib().sv_last_error()


def _problem(spec, seed):
    from eagle_tree_verification_attn_amd.problem import DeviceProblem
    from synth import make_instance
    return DeviceProblem(make_instance(spec, seed), device="cuda:0")


def _results(dev):
    import torch
    torch.cuda.synchronize()
    return {"out": dev.out.view(torch.int16).cpu().numpy() if dev.out.dtype == torch.bfloat16 else dev.out.cpu().numpy(),
            "anc": dev.anc.cpu().numpy(), "depth": dev.depth.cpu().numpy(), "status": dev.status.cpu().numpy(),
            "out_tokens": dev.out_tokens.cpu().numpy(), "out_nodes": dev.out_nodes.cpu().numpy(),
            "out_count": dev.out_count.cpu().numpy(), "out_passes": dev.out_passes.cpu().numpy()}


@pytest.mark.gpu
def test_noalloc_matches_verify_step_twice():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    first = dict(cfg_id=600, B=6, Hq=16, Hkv=2, D=128, dtype="bf16", logit_dtype="bf16",
                 prefix_len=[0, 100, 1500, 33, 640, 2000], tree=("dynamic", 1, 6, 1, 8, 1, 60), V=20000,
                 tau=("choice", [0.0, 0.7, 1.0]), sigma=1.0, draft_std=3.0, sibling_mode="wor")
    second = dict(cfg_id=601, B=3, Hq=8, Hkv=2, D=64, dtype="bf16", logit_dtype="bf16",
                  prefix_len=[300, 0, 90], tree=("widths", [2, 3]), V=5000, tau=0.9, sigma=1.0,
                  draft_std=3.0, sibling_mode="iid")
    old = os.environ.get("SV_ATTN_LSPLIT")
    os.environ["SV_ATTN_LSPLIT"] = "3"      # attention partials in the scratch array too
    try:
        for k, spec in enumerate((first, second)):
            print(f"noalloc call {k}: B={spec['B']} D={spec['D']} V={spec['V']}", flush=True)
            ref_dev = _problem(spec, k)
            ref_dev.verify_step()
            ref = _results(ref_dev)
            dev = _problem(spec, k)
            need = sv.sv_workspace_bytes(dev.tree, dev.attn, dev.acc)
            assert 0 < need <= SCRATCH_BYTES
            sv.sv_verify_step_noalloc(dev.tree, dev.attn, dev.acc, dev.anc, dev.depth, dev.status)
            got = _results(dev)
            for name in ref:
                np.testing.assert_array_equal(got[name], ref[name], err_msg=f"call {k}: {name}")
            assert (ref["status"] == 0).all() and (ref["out_count"] >= 1).all()
    finally:
        if old is None:
            os.environ.pop("SV_ATTN_LSPLIT", None)
        else:
            os.environ["SV_ATTN_LSPLIT"] = old
