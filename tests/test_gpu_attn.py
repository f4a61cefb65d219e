"""GPU tree attention (sv_tree_attn) against the float64 oracle.

Small cases are compared element by element (several key blocks, ragged
prefixes including 0, ragged trees, T_b = 1, every instantiated kernel shape,
forced key splits, the plan made on the device from the trees' actual sizes,
fp32 and bf16).  The five workload shapes run at full size
in the launch configuration the benchmark uses and are compared on every
output element, and so is one GPU's share of the 70B-shaped batch under a 2-
and 8-way KV-head split.  Peaked inputs (queries and keys with std 2, 3, 4, i.e. score
spreads of 4 to 16 in natural units, and one planted dominant key per row on
the row's own tree node, its parent or a prefix key) cover the regime of a
trained target's forward pass, at a short-prefix shape and at the full
Llama-3-70B-shaped batch.
"""
import os

import numpy as np
import pytest

import oracle
from gpu_util import check_attention, need_gpu, say, sv_problem
from synth import CONFIGS, kv_head_shard, make_instance

pytestmark = pytest.mark.gpu


def _spec(**kw):
    s = dict(cfg_id=100, B=2, Hq=8, Hkv=2, D=128, dtype="bf16", logit_dtype="bf16", prefix_len=64,
             tree=("widths", [2, 3]), V=64, tau=1.0, sigma=1.0, draft_std=3.0, sibling_mode="wor")
    s.update(kw)
    return s


def _run(inst, label, env=None, rows=None):
    old = {}
    for k, v in (env or {}).items():
        old[k] = os.environ.get(k)
        os.environ[k] = v
    try:
        say(f"attn {label} B={inst.B} Hq={inst.Hq} Hkv={inst.Hkv} D={inst.D} T_max={inst.T_max} "
            f"L={inst.prefix_len.tolist()} env={env}")
        dev = sv_problem(inst, with_accept=False)
        dev.mask_build()
        dev.tree_attn()
        got = dev.attn_result()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    anc, _, _, status = oracle.tree_mask(inst.parent, inst.num_nodes, inst.T_max)
    ref = oracle.tree_attention(inst.q, inst.k_new, inst.v_new, inst.k_cache, inst.v_cache,
                                inst.prefix_len, anc, inst.num_nodes, status, inst.dtype, units=rows)
    err = check_attention(got, ref, inst.dtype, rows=rows, label=label)
    # rows past each tree are exactly zero
    for b in range(inst.B):
        assert not got[b, int(inst.num_nodes[b]):].any()
    return err


SMALL = {
    "bf16_g8_d128_ragged": _spec(B=3, Hq=16, Hkv=2, prefix_len=[0, 77, 300],
                                 tree=("dynamic", 1, 5, 1, 6, 1, 40), T_max=48),
    "bf16_g8_d64_ragged": _spec(B=3, Hq=16, Hkv=2, D=64, prefix_len=[513, 64, 1],
                                tree=("dynamic", 1, 6, 1, 8, 1, 60)),
    "bf16_chain_g4": _spec(B=4, Hq=8, Hkv=2, prefix_len=[2048, 100, 31, 0], tree=("chain", 4)),
    "bf16_decode_T1": _spec(B=3, Hq=4, Hkv=4, prefix_len=[1, 250, 1000], tree=("chain", 0)),
    "bf16_g5_d128": _spec(B=2, Hq=10, Hkv=2, prefix_len=[333, 1200], tree=("widths", [4, 8, 8])),
    "bf16_g1_d64": _spec(B=2, Hq=3, Hkv=3, D=64, prefix_len=[95, 96], tree=("widths", [2, 2, 2])),
    "bf16_long_prefix": _spec(B=1, Hq=8, Hkv=1, prefix_len=5000, tree=("widths", [3, 4, 5])),
    "f32_tiny": _spec(B=1, Hq=4, Hkv=4, D=64, dtype="f32", prefix_len=128, tree=("widths", [2, 4, 4])),
    "f32_g5_d128_ragged": _spec(B=3, Hq=10, Hkv=2, dtype="f32", prefix_len=[0, 200, 700],
                                tree=("dynamic", 1, 4, 1, 5, 1, 30)),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_attention_small(name):
    need_gpu()
    inst = make_instance(SMALL[name], 1, with_accept=False)
    _run(inst, name)


@pytest.mark.parametrize("variant", ["3,4", "2,4", "2,1", "1,1"])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_every_kernel_shape(variant, D):
    need_gpu()
    if D == 64:
        variant = {"3,4": "4,4", "2,4": "3,4"}.get(variant, variant)
    spec = _spec(B=2, Hq=16, Hkv=2, D=D, prefix_len=[190, 411], tree=("dynamic", 2, 5, 2, 8, 10, 45))
    inst = make_instance(spec, 2, with_accept=False)
    _run(inst, f"shape D={D} {variant}", env={"SV_ATTN_VARIANT": variant})


@pytest.mark.parametrize("lsplit", [2, 3, 7])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_key_splits(lsplit, dtype):
    need_gpu()
    spec = _spec(B=2, Hq=8, Hkv=2, dtype=dtype, prefix_len=[700, 33], tree=("widths", [3, 3, 3]))
    inst = make_instance(spec, 3, with_accept=False)
    _run(inst, f"lsplit={lsplit} {dtype}", env={"SV_ATTN_LSPLIT": str(lsplit)})


@pytest.mark.parametrize("lsplit", [17, 20])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_many_key_splits(lsplit, dtype):
    """More key ranges than the merge loads in its first round trip (16):
    the merge's loop path, with ranges that are empty for the short prefix."""
    need_gpu()
    spec = _spec(B=2, Hq=8, Hkv=2, dtype=dtype, prefix_len=[3000, 45], tree=("widths", [3, 3, 3]))
    inst = make_instance(spec, 5, with_accept=False)
    _run(inst, f"lsplit={lsplit} {dtype}", env={"SV_ATTN_LSPLIT": str(lsplit)})


@pytest.mark.parametrize("lsplit", ["1", "3"])
@pytest.mark.parametrize("D", [128, 64])
def test_attention_odd_kv_heads(D, lsplit):
    """Three KV heads (odd), ragged prefixes including 0, with and without key splits."""
    need_gpu()
    spec = _spec(B=3, Hq=12, Hkv=3, D=D, prefix_len=[300, 0, 97], tree=("dynamic", 2, 5, 2, 6, 5, 40))
    inst = make_instance(spec, 6, with_accept=False)
    _run(inst, f"odd Hkv D={D} lsplit={lsplit}", env={"SV_ATTN_LSPLIT": lsplit})


def test_attention_invalid_sequences_zero():
    need_gpu()
    spec = _spec(B=3, prefix_len=[50, 60, 70], tree=("widths", [2, 2]))
    inst = make_instance(spec, 4, with_accept=False)
    inst.parent[1, 2] = 5          # parent not before its child
    inst.prefix_len[2] = 10_000    # beyond the cache
    say("attn invalid sequences")
    dev = sv_problem(inst, with_accept=False)
    dev.mask_build()
    dev.tree_attn()
    got = dev.attn_result()
    assert np.abs(got[0]).sum() > 0
    assert not got[1].any() and not got[2].any()


@pytest.mark.parametrize("dyn", ["1", "0"])
@pytest.mark.parametrize("D", [128, 64])
def test_attention_sizes_driven_plan(D, dyn, capfd):
    """With key splits and several row blocks per (sequence, KV head), the
    kernel shares out only the row blocks that hold valid rows and picks the
    key split from the trees' actual sizes.  80 sequences (more than one wave
    of 64 counts them), trees of 1 to 40 nodes, prefixes including 0, and two
    invalid sequences (no row blocks); SV_ATTN_DYN=0 keeps the host's plan."""
    need_gpu()
    rng = np.random.default_rng(11)
    B = 80
    prefix = rng.integers(0, 700, size=B).tolist()
    prefix[3] = 0
    spec = _spec(B=B, Hq=8, Hkv=1, D=D, prefix_len=prefix, tree=("dynamic", 1, 5, 1, 6, 1, 40), T_max=40)
    inst = make_instance(spec, 12, with_accept=False)
    big = [b for b in range(B) if inst.num_nodes[b] >= 3]
    inst.parent[big[0], 2] = 7          # parent not before its child
    inst.parent[big[1], 1] = -1         # a second root
    _run(inst, f"sizes-driven plan D={D} dyn={dyn}", env={"SV_ATTN_DYN": dyn, "SV_DEBUG_PLAN": "1"})
    plan = capfd.readouterr().err
    assert f"dyn={dyn}" in plan, plan
    assert "msplit=1 " not in plan and "lsplit=1 " not in plan, plan


@pytest.mark.parametrize("cfg", [c["name"] for c in CONFIGS])
def test_attention_full_workloads(cfg):
    """Every (sequence, position, head) row of each workload at full size."""
    need_gpu()
    spec = dict(next(c for c in CONFIGS if c["name"] == cfg))
    inst = make_instance(spec, 0, with_accept=False)
    _run(inst, f"full {cfg}")


@pytest.mark.parametrize("n", [2, 8])
def test_attention_kv_head_shard(n, capfd):
    """One GPU's share of the Llama-3-70B-shaped batch when the target is
    tensor-parallel over n GPUs: 32 sequences, 64/n query and 8/n KV heads,
    prefix 8192, 65 tree positions.  With one KV head (n = 8) there are only
    32 (sequence, KV head) units, and the plan splits the keys to fill the
    GPU; every output row is compared."""
    need_gpu()
    spec = kv_head_shard("tree64_llama70b_b32", n)
    inst = make_instance(spec, 0, with_accept=False)
    _run(inst, f"kv-head shard 1/{n}", env={"SV_DEBUG_PLAN": "1"})
    plan = capfd.readouterr().err
    if n == 8:
        assert "lsplit=1 " not in plan, plan


@pytest.mark.parametrize("plant", [None, 6.0])
@pytest.mark.parametrize("qk_std", [2.0, 3.0, 4.0])
@pytest.mark.parametrize("D", [128, 64])
def test_attention_peaked(D, qk_std, plant):
    """Large scores: queries and keys N(0, qk_std^2), optionally one planted
    dominant key per row; ragged prefixes (0 included) and ragged trees."""
    need_gpu()
    spec = _spec(B=3, Hq=16, Hkv=2, D=D, prefix_len=[0, 77, 1300], tree=("dynamic", 1, 6, 1, 8, 1, 60),
                 qk_std=qk_std, plant=plant)
    inst = make_instance(spec, 21, with_accept=False)
    _run(inst, f"peaked D={D} std={qk_std} plant={plant}")


@pytest.mark.parametrize("lsplit", ["1", "4"])
def test_attention_peaked_key_splits(lsplit):
    """Peaked scores with the key range split: the partials' offsets and the
    merge carry the large exponents."""
    need_gpu()
    spec = _spec(B=2, Hq=16, Hkv=2, prefix_len=[2000, 333], tree=("widths", [3, 4, 5]), qk_std=3.0, plant=6.0)
    inst = make_instance(spec, 22, with_accept=False)
    _run(inst, f"peaked lsplit={lsplit}", env={"SV_ATTN_LSPLIT": lsplit})


def test_attention_peaked_headline():
    """The Llama-3-70B-shaped batch (32 sequences, 64/8 heads, D = 128, prefix
    8192, 65 tree positions) with queries and keys of std 3 and a planted key
    per row (half of them tree keys), in the benchmark's launch plan; every
    output row compared."""
    need_gpu()
    spec = dict(next(c for c in CONFIGS if c["name"] == "tree64_llama70b_b32"))
    spec.update(qk_std=3.0, plant=6.0)
    inst = make_instance(spec, 3, with_accept=False)
    _run(inst, "peaked headline std=3 plant=6")


def test_attention_from_host_threads():
    """Four host threads, each with its own stream, workspace and outputs, run
    the mask and the attention at the same time; each result equals the one
    the same problem gives in a serial call, bit for bit."""
    need_gpu()
    import threading

    import torch
    specs = [_spec(B=3, Hq=16, Hkv=2, prefix_len=[0, 77, 300], tree=("dynamic", 1, 5, 1, 6, 1, 40), T_max=48),
             _spec(B=3, Hq=16, Hkv=2, D=64, prefix_len=[513, 64, 1], tree=("dynamic", 1, 6, 1, 8, 1, 60)),
             _spec(B=2, Hq=8, Hkv=8, prefix_len=[1000, 129]),
             _spec(B=4, Hq=16, Hkv=2, prefix_len=[2048, 5, 640, 0])]
    insts = [make_instance(s, 10 + i, with_accept=False) for i, s in enumerate(specs)]
    say("attn host threads: serial reference calls")
    serial = []
    for inst in insts:
        dev = sv_problem(inst, with_accept=False)
        dev.mask_build()
        dev.tree_attn()
        serial.append(dev.out.clone())
    torch.cuda.synchronize()
    devs = [sv_problem(inst, with_accept=False) for inst in insts]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            for _ in range(5):
                devs[i].mask_build(stream=s)
                devs[i].tree_attn(stream=s)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {i}: {e}")

    say("attn host threads: 4 threads x 5 calls")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(devs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, dev in enumerate(devs):
        assert torch.equal(dev.out, serial[i]), f"problem {i} differs from its serial result"
