"""Draft-tree verification on MI355X: Python binding of the C ABI in include/sv.h.

This module only marshals arguments: every step of the verification path runs
in the HIP kernels of ``libsv.so``.  Tensors are torch tensors on the GPU; the
binding passes their ``data_ptr()`` and shapes, and the current torch stream
unless a stream is given.  If ``libsv.so`` is missing the import of the
library fails loudly (build it with ``python -m eagle_tree_verification_attn_amd.build``).

Entry points (same names as the C ABI):
    sv_tree_mask_build, sv_tree_attn, sv_spec_accept, sv_verify_step,
    sv_verify_step_noalloc, sv_commit_accepted, sv_workspace_bytes, sv_status_string, sv_last_error
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsv.so")

# ---- constants mirrored from include/sv.h
SV_OK, SV_E_NULL, SV_E_SHAPE, SV_E_DTYPE, SV_E_WORKSPACE, SV_E_HIP, SV_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
SV_TREE_OK, SV_TREE_E_ROOT, SV_TREE_E_PARENT, SV_TREE_E_COUNT = 0, 1, 2, 3
SV_TREE_E_TOKEN, SV_TREE_E_NONFINITE, SV_TREE_E_NOQ, SV_TREE_E_SYNC = 4, 5, 6, 7
SV_TREE_E_CACHE, SV_TREE_E_PATH, SV_TREE_E_PROB = 8, 9, 10
SV_F32, SV_BF16 = 0, 1
SV_SIB_WITHOUT_REPLACEMENT, SV_SIB_IID = 0, 1

EXPORTS = ["sv_tree_mask_build", "sv_tree_attn", "sv_spec_accept", "sv_verify_step", "sv_verify_step_noalloc",
           "sv_commit_accepted", "sv_workspace_bytes", "sv_status_string", "sv_last_error",
           "sv_eagle2_state_bytes", "sv_eagle2_begin", "sv_eagle2_expand", "sv_eagle2_finish",
           "sv_eagle2_expand_finish", "sv_draft_head"]


class SvTree(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T_max", ctypes.c_int32), ("parent", ctypes.c_void_p),
                ("num_nodes", ctypes.c_void_p), ("tokens", ctypes.c_void_p)]


class SvAttnArgs(ctypes.Structure):
    _fields_ = [("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("L_max", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("prefix_len", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class SvAcceptArgs(ctypes.Structure):
    _fields_ = [("V", ctypes.c_int32), ("logit_dtype", ctypes.c_int32),
                ("sibling_mode", ctypes.c_int32), ("target_logits", ctypes.c_void_p),
                ("q_probs", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
                ("u_accept", ctypes.c_void_p), ("u_sample", ctypes.c_void_p),
                ("out_tokens", ctypes.c_void_p), ("out_nodes", ctypes.c_void_p),
                ("out_count", ctypes.c_void_p), ("out_passes", ctypes.c_void_p)]


class SvEagle2Cfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("V", ctypes.c_int32), ("k", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("m", ctypes.c_int32)]


class SvHeadArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("d", ctypes.c_int32), ("r", ctypes.c_int32), ("n", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("k_tile", ctypes.c_int32), ("h", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("A_sh", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("W", ctypes.c_void_p), ("u", ctypes.c_void_p),
                ("cand_ids", ctypes.c_void_p), ("cand_logits", ctypes.c_void_p)]


class SvCommitArgs(ctypes.Structure):
    _fields_ = [("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("L_max", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("prefix_len", ctypes.c_void_p), ("prefix_len_out", ctypes.c_void_p),
                ("F", ctypes.c_int32), ("feat_dtype", ctypes.c_int32),
                ("feat_in", ctypes.c_void_p), ("feat_out", ctypes.c_void_p)]


class SvError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {sv_status_string(code)} ({code}): {sv_last_error()}")


_lib = None


def lib():
    """The loaded libsv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m eagle_tree_verification_attn_amd.build`")
        # torch ships its own HIP runtime under the same soname as the system
        # one libsv.so is linked against.  Loaded first, torch's runtime
        # satisfies libsv.so's dependency, so the process has one runtime and
        # torch's streams and memory are valid in the library.  Loaded the
        # other way round, the process would get two runtimes and torch would
        # find no GPU.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.sv_tree_mask_build.argtypes = [P(SvTree), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.sv_tree_attn.argtypes = [P(SvTree), ctypes.c_void_p, ctypes.c_void_p, P(SvAttnArgs),
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.sv_spec_accept.argtypes = [P(SvTree), ctypes.c_void_p, P(SvAcceptArgs), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
        L.sv_verify_step.argtypes = [P(SvTree), P(SvAttnArgs), P(SvAcceptArgs), ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
        L.sv_verify_step_noalloc.argtypes = [P(SvTree), P(SvAttnArgs), P(SvAcceptArgs), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.sv_commit_accepted.argtypes = [P(SvTree), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         P(SvCommitArgs), ctypes.c_void_p]
        L.sv_eagle2_state_bytes.argtypes = [P(SvEagle2Cfg)]
        L.sv_eagle2_state_bytes.restype = ctypes.c_size_t
        L.sv_eagle2_begin.argtypes = [P(SvEagle2Cfg), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_void_p]
        L.sv_eagle2_expand.argtypes = [P(SvEagle2Cfg), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.sv_eagle2_finish.argtypes = [P(SvEagle2Cfg), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.sv_eagle2_expand_finish.argtypes = [P(SvEagle2Cfg), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.sv_draft_head.argtypes = [P(SvHeadArgs), ctypes.c_void_p]
        L.sv_workspace_bytes.argtypes = [P(SvTree), P(SvAttnArgs), P(SvAcceptArgs)]
        L.sv_workspace_bytes.restype = ctypes.c_size_t
        L.sv_status_string.argtypes = [ctypes.c_int32]
        L.sv_status_string.restype = ctypes.c_char_p
        L.sv_last_error.argtypes = []
        L.sv_last_error.restype = ctypes.c_char_p
        for f in ("sv_tree_mask_build", "sv_tree_attn", "sv_spec_accept", "sv_verify_step", "sv_verify_step_noalloc",
                  "sv_commit_accepted",
                  "sv_eagle2_begin", "sv_eagle2_expand", "sv_eagle2_finish", "sv_eagle2_expand_finish",
                  "sv_draft_head"):
            getattr(L, f).restype = ctypes.c_int32
        _lib = L
    return _lib


# ---------------------------------------------------------------- marshalling
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_tree(parent, num_nodes, tokens=None):
    """sv_tree from int32 device tensors parent [B][T_max], num_nodes [B], tokens [B][T_max]."""
    B, T_max = (int(parent.shape[0]), int(parent.shape[1])) if parent is not None else (0, 1)
    t = SvTree(B, T_max, _ptr(parent), _ptr(num_nodes), _ptr(tokens))
    t._keep = (parent, num_nodes, tokens)
    return t


def make_attn_args(q, k_new, v_new, k_cache, v_cache, prefix_len, out, scale=0.0):
    """sv_attn_args: q [B][T_max][Hq][D], k_new/v_new [B][T_max][Hkv][D],
    k_cache/v_cache [B][Hkv][L_max][D], prefix_len int32 [B], out like q."""
    Hq, D = int(q.shape[2]), int(q.shape[3])
    Hkv = int(k_new.shape[2])
    L_max = int(k_cache.shape[2])
    a = SvAttnArgs(Hq, Hkv, D, L_max, _dtype_code(q), float(scale), _ptr(q), _ptr(k_new),
                   _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(out))
    a._keep = (q, k_new, v_new, k_cache, v_cache, prefix_len, out)
    return a


def make_accept_args(target_logits, q_probs, temperature, u_accept, u_sample, out_tokens,
                     out_nodes, out_count, out_passes=None, sibling_mode=SV_SIB_WITHOUT_REPLACEMENT):
    """sv_accept_args: target_logits [B][T_max][V] (fp32 or bf16), q_probs fp32 or None,
    temperature/u_accept/u_sample fp32, outputs int32."""
    V = int(target_logits.shape[2])
    a = SvAcceptArgs(V, _dtype_code(target_logits), int(sibling_mode), _ptr(target_logits),
                     _ptr(q_probs), _ptr(temperature), _ptr(u_accept), _ptr(u_sample),
                     _ptr(out_tokens), _ptr(out_nodes), _ptr(out_count), _ptr(out_passes))
    a._keep = (target_logits, q_probs, temperature, u_accept, u_sample, out_tokens, out_nodes,
               out_count, out_passes)
    return a


def make_commit_args(k_new, v_new, k_cache, v_cache, prefix_len, prefix_len_out, feat_in=None, feat_out=None):
    """sv_commit_args: k_new/v_new [B][T_max][Hkv][D], k_cache/v_cache [B][Hkv][L_max][D],
    prefix_len / prefix_len_out int32 [B], optional feat_in / feat_out [B][T_max][F]."""
    Hkv, D = int(k_new.shape[2]), int(k_new.shape[3])
    L_max = int(k_cache.shape[2])
    F = 0 if feat_in is None else int(feat_in.shape[2])
    fdt = SV_F32 if feat_in is None else _dtype_code(feat_in)
    a = SvCommitArgs(Hkv, D, L_max, _dtype_code(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                     _ptr(prefix_len), _ptr(prefix_len_out), F, fdt, _ptr(feat_in), _ptr(feat_out))
    a._keep = (k_new, v_new, k_cache, v_cache, prefix_len, prefix_len_out, feat_in, feat_out)
    return a


def _check(code, where, raise_on_error):
    if code != SV_OK and raise_on_error:
        raise SvError(code, where)
    return code


# ---------------------------------------------------------------- entry points
def sv_tree_mask_build(tree, anc, depth, tree_status, stream=None, raise_on_error=True):
    return _check(lib().sv_tree_mask_build(ctypes.byref(tree), _ptr(anc), _ptr(depth), _ptr(tree_status),
                                           _stream(stream)), "sv_tree_mask_build", raise_on_error)


def sv_tree_attn(tree, anc, tree_status, attn, ws, stream=None, raise_on_error=True):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return _check(lib().sv_tree_attn(ctypes.byref(tree), _ptr(anc), _ptr(tree_status), ctypes.byref(attn),
                                     _ptr(ws), nbytes, _stream(stream)), "sv_tree_attn", raise_on_error)


def sv_spec_accept(tree, tree_status, acc, ws, stream=None, raise_on_error=True):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return _check(lib().sv_spec_accept(ctypes.byref(tree), _ptr(tree_status), ctypes.byref(acc), _ptr(ws),
                                       nbytes, _stream(stream)), "sv_spec_accept", raise_on_error)


def sv_verify_step(tree, attn, acc, anc, depth, tree_status, ws, stream=None, raise_on_error=True):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return _check(lib().sv_verify_step(ctypes.byref(tree), ctypes.byref(attn), ctypes.byref(acc), _ptr(anc),
                                       _ptr(depth), _ptr(tree_status), _ptr(ws), nbytes, _stream(stream)),
                  "sv_verify_step", raise_on_error)


def sv_verify_step_noalloc(tree, attn, acc, anc, depth, tree_status, stream=None, raise_on_error=True):
    return _check(lib().sv_verify_step_noalloc(ctypes.byref(tree), ctypes.byref(attn), ctypes.byref(acc), _ptr(anc),
                                               _ptr(depth), _ptr(tree_status), _stream(stream)),
                  "sv_verify_step_noalloc", raise_on_error)


def sv_commit_accepted(tree, tree_status, out_nodes, out_count, commit, stream=None, raise_on_error=True):
    return _check(lib().sv_commit_accepted(ctypes.byref(tree), _ptr(tree_status), _ptr(out_nodes), _ptr(out_count),
                                           ctypes.byref(commit), _stream(stream)),
                  "sv_commit_accepted", raise_on_error)


def sv_eagle2_state_bytes(cfg):
    return int(lib().sv_eagle2_state_bytes(ctypes.byref(cfg)))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def sv_eagle2_begin(cfg, state, root_tokens, stream=None, raise_on_error=True):
    return _check(lib().sv_eagle2_begin(ctypes.byref(cfg), _ptr(state), _nbytes(state), _ptr(root_tokens),
                                        _stream(stream)), "sv_eagle2_begin", raise_on_error)


def sv_eagle2_expand(cfg, state, step, q, frontier=None, frontier_tokens=None, stream=None, raise_on_error=True):
    return _check(lib().sv_eagle2_expand(ctypes.byref(cfg), _ptr(state), _nbytes(state), int(step), _ptr(q),
                                         _ptr(frontier), _ptr(frontier_tokens), _stream(stream)),
                  "sv_eagle2_expand", raise_on_error)


def sv_eagle2_finish(cfg, state, parent, tokens, num_nodes, q_row, status, stream=None, raise_on_error=True):
    return _check(lib().sv_eagle2_finish(ctypes.byref(cfg), _ptr(state), _nbytes(state), _ptr(parent), _ptr(tokens),
                                         _ptr(num_nodes), _ptr(q_row), _ptr(status), _stream(stream)),
                  "sv_eagle2_finish", raise_on_error)


def sv_eagle2_expand_finish(cfg, state, step, q, parent, tokens, num_nodes, q_row, status, stream=None,
                            raise_on_error=True):
    return _check(lib().sv_eagle2_expand_finish(ctypes.byref(cfg), _ptr(state), _nbytes(state), int(step), _ptr(q),
                                                _ptr(parent), _ptr(tokens), _ptr(num_nodes), _ptr(q_row),
                                                _ptr(status), _stream(stream)),
                  "sv_eagle2_expand_finish", raise_on_error)


def make_head_args(h, B, A_sh, perm, W, u, cand_ids, cand_logits, tile, k_tile):
    """sv_head_args: h [N][d], B [r][d], A_sh [n][r], W [n][d] bf16; perm [n] int32; outputs u [N][r] bf16,
    cand_ids int32 / cand_logits fp32 [N][ceil(n / tile) * k_tile]."""
    N, d = int(h.shape[0]), int(h.shape[1])
    r, n = int(B.shape[0]), int(A_sh.shape[0])
    a = SvHeadArgs(N, d, r, n, int(tile), int(k_tile), _ptr(h), _ptr(B), _ptr(A_sh), _ptr(perm), _ptr(W), _ptr(u),
                   _ptr(cand_ids), _ptr(cand_logits))
    a._keep = (h, B, A_sh, perm, W, u, cand_ids, cand_logits)
    return a


def sv_draft_head(args, stream=None, raise_on_error=True):
    return _check(lib().sv_draft_head(ctypes.byref(args), _stream(stream)), "sv_draft_head", raise_on_error)


def sv_workspace_bytes(tree, attn=None, acc=None):
    return int(lib().sv_workspace_bytes(ctypes.byref(tree), ctypes.byref(attn) if attn is not None else None,
                                        ctypes.byref(acc) if acc is not None else None))


def sv_status_string(code):
    return lib().sv_status_string(int(code)).decode()


def sv_last_error():
    return lib().sv_last_error().decode()
