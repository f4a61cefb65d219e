"""Device-side buffers for one verification problem (argument marshalling).

``DeviceProblem`` uploads host arrays (NumPy; bf16 data as uint16 bit
patterns) to torch tensors on the GPU, allocates the outputs and the workspace,
and builds the C-ABI structs.  Its methods call the library's entry points on
the current torch stream.  Nothing here computes any part of the verification.
"""
import numpy as np

from . import (SV_SIB_IID, SV_SIB_WITHOUT_REPLACEMENT, SvEagle2Cfg, make_accept_args, make_attn_args,
               make_commit_args, make_tree, sv_commit_accepted, sv_eagle2_begin, sv_eagle2_expand,
               sv_eagle2_expand_finish, sv_eagle2_finish,
               sv_eagle2_state_bytes, sv_spec_accept, sv_tree_attn, sv_tree_mask_build, sv_verify_step,
               sv_workspace_bytes)


def to_device(arr, dtype, device):
    """NumPy -> torch on ``device``; dtype 'bf16' reads uint16 bit patterns."""
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def bf16_bits(t):
    """torch bfloat16 tensor -> NumPy uint16 bit patterns (host)."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceProblem:
    """Inputs, outputs and workspace of one batch on one GPU.

    ``src`` is any object with the attributes of a problem instance: B, T_max,
    parent, num_nodes, tokens, and for attention q, k_new, v_new, k_cache,
    v_cache, prefix_len, dtype; for acceptance target_logits, logit_dtype,
    q_probs, temperature, u_accept, u_sample, sibling_mode.
    """

    def __init__(self, src, device="cuda", with_attn=True, with_accept=True, scale=0.0):
        import torch
        self.device = device
        B, T = int(src.B), int(src.T_max)
        self.B, self.T_max = B, T
        i32 = lambda a: to_device(np.asarray(a, dtype=np.int32), "i32", device)
        self.parent = i32(src.parent)
        self.num_nodes = i32(src.num_nodes)
        self.tokens = i32(src.tokens)
        self.tree = make_tree(self.parent, self.num_nodes, self.tokens)
        W = (T + 63) // 64
        self.anc = torch.zeros((B, T, W), dtype=torch.int64, device=device)
        self.depth = torch.zeros((B, T), dtype=torch.int32, device=device)
        self.status = torch.zeros((B,), dtype=torch.int32, device=device)
        self.attn = None
        self.acc = None
        if with_attn and getattr(src, "q", None) is not None:
            dt = src.dtype
            self.q = to_device(src.q, dt, device)
            self.k_new = to_device(src.k_new, dt, device)
            self.v_new = to_device(src.v_new, dt, device)
            self.k_cache = to_device(src.k_cache, dt, device)
            self.v_cache = to_device(src.v_cache, dt, device)
            self.prefix_len = i32(src.prefix_len)
            self.out = torch.empty_like(self.q)
            self.attn = make_attn_args(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache,
                                       self.prefix_len, self.out, scale)
        if with_accept and getattr(src, "target_logits", None) is not None:
            self.logits = to_device(src.target_logits, src.logit_dtype, device)
            self.q_probs = None if src.q_probs is None else to_device(src.q_probs, "f32", device)
            self.temperature = to_device(np.asarray(src.temperature, dtype=np.float32), "f32", device)
            self.u_accept = to_device(np.asarray(src.u_accept, dtype=np.float32), "f32", device)
            self.u_sample = to_device(np.asarray(src.u_sample, dtype=np.float32), "f32", device)
            self.out_tokens = torch.full((B, T), -7, dtype=torch.int32, device=device)
            self.out_nodes = torch.full((B, T), -7, dtype=torch.int32, device=device)
            self.out_count = torch.full((B,), -7, dtype=torch.int32, device=device)
            self.out_passes = torch.full((B,), -7, dtype=torch.int32, device=device)
            mode = SV_SIB_IID if getattr(src, "sibling_mode", "wor") == "iid" else SV_SIB_WITHOUT_REPLACEMENT
            self.acc = make_accept_args(self.logits, self.q_probs, self.temperature, self.u_accept,
                                        self.u_sample, self.out_tokens, self.out_nodes, self.out_count,
                                        self.out_passes, mode)
        nbytes = sv_workspace_bytes(self.tree, self.attn, self.acc)
        self.ws = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)

    # ---- entry points on this problem
    def mask_build(self, stream=None):
        return sv_tree_mask_build(self.tree, self.anc, self.depth, self.status, stream)

    def tree_attn(self, stream=None):
        return sv_tree_attn(self.tree, self.anc, self.status, self.attn, self.ws, stream)

    def spec_accept(self, stream=None):
        return sv_spec_accept(self.tree, self.status, self.acc, self.ws, stream)

    def verify_step(self, stream=None):
        return sv_verify_step(self.tree, self.attn, self.acc, self.anc, self.depth, self.status,
                              self.ws, stream)

    def commit_args(self, feat_in=None):
        """Commit arguments writing into this problem's caches; new lengths go to
        ``self.prefix_len_out`` and features (optional [B][T_max][F] tensor) to
        ``self.feat_out``."""
        import torch
        self.prefix_len_out = torch.full_like(self.prefix_len, -7)
        self.feat_in = feat_in
        self.feat_out = None if feat_in is None else torch.full_like(feat_in, 7.0)
        self.commit = make_commit_args(self.k_new, self.v_new, self.k_cache, self.v_cache, self.prefix_len,
                                       self.prefix_len_out, self.feat_in, self.feat_out)
        return self.commit

    def commit_accepted(self, stream=None):
        return sv_commit_accepted(self.tree, self.status, self.out_nodes, self.out_count, self.commit, stream)

    # ---- results on the host
    def mask_results(self):
        return (self.anc.cpu().numpy().view(np.uint64), self.depth.cpu().numpy(),
                self.status.cpu().numpy())

    def attn_result(self):
        """Attention output as float64 on the host."""
        import torch
        return self.out.to(torch.float64).cpu().numpy()

    def accept_results(self):
        return dict(out_nodes=self.out_nodes.cpu().numpy(), out_tokens=self.out_tokens.cpu().numpy(),
                    out_count=self.out_count.cpu().numpy(), out_passes=self.out_passes.cpu().numpy(),
                    status=self.status.cpu().numpy())


class DeviceTreeBuilder:
    """State and outputs of the EAGLE-2 tree builder for one batch on one GPU.

    ``run(q_steps, root_tokens)`` takes one device float32 tensor [B][k][V] per
    expansion step (the drafter's probability rows for that step's frontier)
    and calls begin, expand for every step and finish on the current stream.
    """

    def __init__(self, B, V, k, depth, m, device="cuda"):
        import torch
        self.cfg = SvEagle2Cfg(B, V, k, depth, m)
        n = sv_eagle2_state_bytes(self.cfg)
        if n == 0:
            raise ValueError("unsupported tree-builder configuration")
        self.state = torch.empty((n,), dtype=torch.uint8, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        T = m + 1
        self.frontier = torch.full((depth, B, k), -7, **i32)
        self.frontier_tokens = torch.full((depth, B, k), -7, **i32)
        self.parent = torch.full((B, T), -7, **i32)
        self.tokens = torch.full((B, T), -7, **i32)
        self.q_row = torch.full((B, T), -7, **i32)
        self.num_nodes = torch.full((B,), -7, **i32)
        self.status = torch.full((B,), -7, **i32)

    def run(self, q_steps, root_tokens, stream=None, fused_last=False):
        """fused_last: the last step and the finish in one call
        (sv_eagle2_expand_finish); that step's frontier is then not written."""
        sv_eagle2_begin(self.cfg, self.state, root_tokens, stream)
        last = self.cfg.depth - 1
        for s in range(self.cfg.depth if not fused_last else last):
            sv_eagle2_expand(self.cfg, self.state, s, q_steps[s], self.frontier[s], self.frontier_tokens[s], stream)
        if fused_last:
            sv_eagle2_expand_finish(self.cfg, self.state, last, q_steps[last], self.parent, self.tokens,
                                    self.num_nodes, self.q_row, self.status, stream)
        else:
            sv_eagle2_finish(self.cfg, self.state, self.parent, self.tokens, self.num_nodes, self.q_row, self.status,
                             stream)

    def results(self):
        return dict(parent=self.parent.cpu().numpy(), tokens=self.tokens.cpu().numpy(),
                    q_row=self.q_row.cpu().numpy(), num_nodes=self.num_nodes.cpu().numpy(),
                    status=self.status.cpu().numpy(), frontier=self.frontier.cpu().numpy(),
                    frontier_tokens=self.frontier_tokens.cpu().numpy())
