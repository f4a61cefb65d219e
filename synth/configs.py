"""The five workload shapes of the verification step, plus small test shapes.

Each spec is a plain dict read by :func:`synth.gen.make_instance`:

``B, Hq, Hkv, D``      batch, query heads, KV heads, head dim
``dtype``              "f32" or "bf16" for q, k, v, cache and attention output
``logit_dtype``        "f32" or "bf16" for the target logits
``prefix_len``         int (same for all sequences) or list of B ints (ragged)
``tree``               ("widths", [w1, w2, ...]) same shape for every sequence,
                       ("chain", N), or ("dynamic", depth_lo, depth_hi, width_lo,
                       width_hi, n_lo, n_hi) drawn per sequence
``V``                  vocabulary size
``tau``                float or list of B floats (0 = greedy)
``sigma``              std of the target-logit noise: z_p = z_q + N(0, sigma^2)
``draft_std``          std of the draft logits z_q ~ N(0, draft_std^2)
``sibling_mode``       "wor" (siblings drawn without replacement) or "iid"
"""

CONFIGS = [
    dict(name="tiny_f32", cfg_id=1, B=1, Hq=4, Hkv=4, D=64, dtype="f32", logit_dtype="f32",
         prefix_len=128, tree=("widths", [2, 4, 4]), V=1000, tau=1.0, sigma=1.0,
         draft_std=3.0, sibling_mode="wor"),
    dict(name="chain_greedy_llama8b", cfg_id=2, B=8, Hq=32, Hkv=8, D=128, dtype="bf16",
         logit_dtype="bf16", prefix_len=2048, tree=("chain", 4), V=128256, tau=0.0,
         sigma=0.7, draft_std=3.0, sibling_mode="wor"),
    dict(name="static_tree_gptoss120b", cfg_id=3, B=8, Hq=64, Hkv=8, D=64, dtype="bf16",
         logit_dtype="bf16", prefix_len=4096, tree=("widths", [4, 8, 12, 12, 12, 12]),
         V=201088, tau=1.0, sigma=1.0, draft_std=3.0, sibling_mode="wor"),
    dict(name="tree64_llama70b_b32", cfg_id=4, B=32, Hq=64, Hkv=8, D=128, dtype="bf16",
         logit_dtype="bf16", prefix_len=8192, tree=("widths", [4, 8, 12, 12, 14, 14]),
         V=128256, tau=0.8, sigma=1.0, draft_std=3.0, sibling_mode="wor"),
    dict(name="long_ctx_dynamic", cfg_id=5, B=4, Hq=40, Hkv=8, D=128, dtype="bf16",
         logit_dtype="bf16", prefix_len=32768, tree=("dynamic", 2, 8, 1, 24, 32, 128),
         V=151936, tau=("choice", [0.0, 0.7, 1.0]), sigma=1.0, draft_std=3.0,
         sibling_mode="wor"),
]


def config_by_name(name):
    for c in CONFIGS:
        if c["name"] == name or str(c["cfg_id"]) == str(name):
            return dict(c)
    raise KeyError(name)


def small_spec(base, **over):
    """A copy of a config spec with some fields replaced (for tests)."""
    s = dict(config_by_name(base) if isinstance(base, (str, int)) else base)
    s.update(over)
    return s


def kv_head_shard(base, n):
    """One GPU's share of a workload whose target model is tensor-parallel over
    n GPUs.  Attention then shards by KV head: each GPU holds Hkv / n KV heads
    and their Hq / n query heads, with every sequence, prefix and tree
    unchanged.  The inputs are drawn for that shape from the workload's own
    seeds."""
    s = dict(config_by_name(base) if isinstance(base, (str, int)) else base)
    if n < 1 or s["Hkv"] % n:
        raise ValueError(f"{s['name']}: {s['Hkv']} KV heads do not split {n} ways")
    if n > 1:
        s["Hq"] //= n
        s["Hkv"] //= n
        s["name"] = f"{s['name']}_kvshard{n}"
    return s
