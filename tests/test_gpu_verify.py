"""The whole step (sv_verify_step: mask -> attention -> accept on one stream,
one workspace) against the oracle, and its repeatability."""
import os

import pytest

import oracle
from gpu_util import check_accept, check_attention, check_mask, need_gpu, say, sv_problem
from synth import CONFIGS, make_instance

pytestmark = pytest.mark.gpu


def _step(inst, label):
    say(f"verify_step {label} B={inst.B} T_max={inst.T_max} V={inst.V}")
    dev = sv_problem(inst)
    dev.verify_step()
    check_mask(dev, inst)
    ref = oracle.verify_step(inst)
    check_attention(dev.attn_result(), ref["attn"], inst.dtype, label=label)
    exempt = check_accept(dev.accept_results(), ref["accept"], label)
    return dev, exempt


@pytest.mark.parametrize("cfg", ["tiny_f32", "chain_greedy_llama8b"])
def test_verify_step_workloads(cfg):
    need_gpu()
    inst = make_instance(dict(next(c for c in CONFIGS if c["name"] == cfg)), 0)
    _step(inst, cfg)


def test_verify_step_headline():
    """The call the benchmark times, at its size: sv_verify_step on the
    32-sequence 70B-shaped workload (the same launch plan); every sequence's
    accept results and every attention output row against the oracle."""
    need_gpu()
    spec = dict(next(c for c in CONFIGS if c["name"] == "tree64_llama70b_b32"))
    inst = make_instance(spec, 0)
    say(f"verify_step headline B={inst.B} T_max={inst.T_max} V={inst.V}")
    dev = sv_problem(inst)
    dev.verify_step()
    check_mask(dev, inst)
    ref = oracle.verify_step(inst)
    check_attention(dev.attn_result(), ref["attn"], inst.dtype, label="headline")
    exempt = check_accept(dev.accept_results(), ref["accept"], "headline")
    say(f"  counts {dev.accept_results()['out_count'].tolist()} exempt {exempt}")


def test_verify_step_mixed_small():
    need_gpu()
    spec = dict(cfg_id=400, B=5, Hq=16, Hkv=2, D=128, dtype="bf16", logit_dtype="bf16",
                prefix_len=[0, 100, 1000, 33, 64], tree=("dynamic", 1, 6, 1, 8, 1, 60), V=9000,
                tau=("choice", [0.0, 0.7, 1.0]), sigma=1.0, draft_std=3.0, sibling_mode="wor")
    inst = make_instance(spec, 3)
    _step(inst, "mixed_small")


def test_verify_step_repeatable():
    need_gpu()
    import torch
    spec = dict(cfg_id=401, B=4, Hq=16, Hkv=2, D=128, dtype="bf16", logit_dtype="bf16",
                prefix_len=[300, 700, 50, 1200], tree=("widths", [4, 8, 8]), V=12000, tau=0.8,
                sigma=1.0, draft_std=3.0, sibling_mode="wor")
    inst = make_instance(spec, 1)
    say("verify_step repeat")
    dev = sv_problem(inst)
    dev.verify_step()
    first = (dev.out.clone(), dev.out_tokens.clone(), dev.out_nodes.clone(), dev.out_count.clone())
    for _ in range(3):
        dev.verify_step()
        assert torch.equal(dev.out.view(torch.int16), first[0].view(torch.int16))
        assert torch.equal(dev.out_tokens, first[1]) and torch.equal(dev.out_nodes, first[2])
        assert torch.equal(dev.out_count, first[3])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_verify_step_split_keys(dtype):
    """Key ranges split four ways: the attention's partial results and the
    walk's exchange words share the step's workspace (the words after the
    partials, zeroed by the mask kernel)."""
    need_gpu()
    spec = dict(cfg_id=402, B=3, Hq=8, Hkv=2, D=64, dtype=dtype, logit_dtype="bf16" if dtype == "bf16" else "f32",
                prefix_len=[900, 0, 2500], tree=("widths", [3, 6, 6]), V=7000, tau=("choice", [0.0, 0.9]),
                sigma=1.0, draft_std=3.0, sibling_mode="wor")
    inst = make_instance(spec, 2)
    old = os.environ.get("SV_ATTN_LSPLIT")
    os.environ["SV_ATTN_LSPLIT"] = "4"
    try:
        _step(inst, f"split keys {dtype}")
    finally:
        if old is None:
            os.environ.pop("SV_ATTN_LSPLIT", None)
        else:
            os.environ["SV_ATTN_LSPLIT"] = old
