"""The C-ABI library: it loads, exports every entry point include/sv.h
declares, mirrors the header's constants, and rejects bad host arguments
before launching anything (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import eagle_tree_verification_attn_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:sv_status|size_t|const char\*)\s+(sv_\w+)\(", text, re.M)))


def _enums():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(SV_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert names == sorted(sv.EXPORTS)
    L = ctypes.CDLL(sv.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", sv.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(r"\bT " + n + r"\b", dyn), n


def test_binding_constants_match_header():
    for k, v in _enums().items():
        assert getattr(sv, k) == v, k


def test_status_strings():
    for code in list(range(-6, 1)) + list(range(1, 11)):
        s = sv.sv_status_string(code)
        assert s and s != "unknown status"
    assert sv.sv_status_string(99) == "unknown status"


def _tree(B=2, T=5):
    fake = ctypes.c_void_p(0x1000)
    t = sv.SvTree(B, T, fake, fake, fake)
    return t


def _attn(**kw):
    fake = 0x10000
    a = sv.SvAttnArgs(8, 2, 64, 16, sv.SV_BF16, 0.0, fake, fake, fake, fake, fake, fake, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _acc(**kw):
    fake = 0x10000
    a = sv.SvAcceptArgs(1000, sv.SV_BF16, 0, fake, fake, fake, fake, fake, fake, fake, fake, None)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_host_validation_rejects_before_launch():
    L = sv.lib()
    null = None
    fake = ctypes.c_void_p(0x10000)
    assert L.sv_tree_mask_build(null, fake, fake, fake, null) == sv.SV_E_NULL
    assert L.sv_tree_mask_build(ctypes.byref(_tree(T=0)), fake, fake, fake, null) == sv.SV_E_SHAPE
    assert L.sv_tree_mask_build(ctypes.byref(_tree(T=257)), fake, fake, fake, null) == sv.SV_E_UNSUPPORTED
    assert L.sv_tree_mask_build(ctypes.byref(_tree(B=-1)), fake, fake, fake, null) == sv.SV_E_SHAPE
    assert L.sv_tree_mask_build(ctypes.byref(_tree()), null, fake, fake, null) == sv.SV_E_NULL
    t = ctypes.byref(_tree())
    assert L.sv_tree_attn(t, fake, fake, ctypes.byref(_attn(Hkv=3)), fake, 1 << 30, null) == sv.SV_E_SHAPE
    assert L.sv_tree_attn(t, fake, fake, ctypes.byref(_attn(D=96)), fake, 1 << 30, null) == sv.SV_E_UNSUPPORTED
    assert L.sv_tree_attn(t, fake, fake, ctypes.byref(_attn(dtype=7)), fake, 1 << 30, null) == sv.SV_E_DTYPE
    assert L.sv_tree_attn(t, fake, fake, ctypes.byref(_attn(q=None)), fake, 1 << 30, null) == sv.SV_E_NULL
    assert L.sv_tree_attn(t, fake, fake, ctypes.byref(_attn(q=0x10008)), fake, 1 << 30, null) == sv.SV_E_UNSUPPORTED
    # 32-bit key offsets: (L_max + 256) * D must stay below 2^31
    big = (1 << 31) // 64 - 256
    assert L.sv_tree_attn(t, fake, fake, ctypes.byref(_attn(L_max=big)), fake, 1 << 30, null) == sv.SV_E_UNSUPPORTED
    assert b"too large for D" in L.sv_last_error()
    assert L.sv_tree_attn(t, fake, fake, ctypes.byref(_attn(L_max=big - 1, q=None)), fake, 1 << 30, null) == sv.SV_E_NULL
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc(V=0)), fake, 1 << 30, null) == sv.SV_E_SHAPE
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc(logit_dtype=5)), fake, 1 << 30, null) == sv.SV_E_DTYPE
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc(sibling_mode=2)), fake, 1 << 30, null) == sv.SV_E_SHAPE
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc(u_sample=None)), fake, 1 << 30, null) == sv.SV_E_NULL
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc(V=2_000_000)), fake, 1 << 30, null) == sv.SV_E_UNSUPPORTED
    # workspace: missing, too small, misaligned
    need = L.sv_workspace_bytes(t, None, ctypes.byref(_acc()))
    assert need > 0
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc()), None, need, null) == sv.SV_E_WORKSPACE
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc()), fake, need - 1, null) == sv.SV_E_WORKSPACE
    assert L.sv_spec_accept(t, fake, ctypes.byref(_acc()), ctypes.c_void_p(0x10010), need, null) == sv.SV_E_WORKSPACE
    assert "workspace" in sv.sv_last_error()
    # an empty batch is valid and launches nothing
    empty = sv.SvTree(0, 4, None, None, None)
    assert L.sv_tree_mask_build(ctypes.byref(empty), None, None, None, null) == sv.SV_OK
    assert sv.sv_last_error() == ""


def test_workspace_sizes_for_the_workloads():
    from synth import CONFIGS
    for c in CONFIGS:
        T = 130 if c["tree"][0] == "dynamic" else 1 + (c["tree"][1] if c["tree"][0] == "chain" else sum(c["tree"][1]))
        t = sv.SvTree(c["B"], T, None, None, None)
        a = _attn(Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], L_max=c["prefix_len"],
                  dtype=sv.SV_BF16 if c["dtype"] == "bf16" else sv.SV_F32)
        acc = _acc(V=c["V"])
        n_acc = sv.sv_workspace_bytes(t, None, acc)
        n_attn = sv.sv_workspace_bytes(t, a, None)
        n_both = sv.sv_workspace_bytes(t, a, acc)
        assert n_acc > 0 and n_both >= n_acc
        assert n_both % 256 == 0
        # the step's layout: the accept's words after the attention's partial results
        assert n_both == -(-n_attn // 256) * 256 + n_acc


# ---------------------------------------------------------------- tree builder (host checks only)
def _e2(**kw):
    c = sv.SvEagle2Cfg(4, 1000, 8, 6, 64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_eagle2_state_bytes_and_config_checks():
    n = sv.sv_eagle2_state_bytes(_e2())
    assert n > 0 and n % 256 == 0
    # nodes before the rerank: 1 + k + (depth-1) k^2
    assert sv.sv_eagle2_state_bytes(_e2(m=255)) > 0                 # 256 verify positions
    assert sv.sv_eagle2_state_bytes(_e2(k=2, depth=2, m=6)) > 0      # all 2 + 4 generated nodes
    for bad in (dict(k=0), dict(k=17), dict(V=4, k=8), dict(m=0), dict(k=2, depth=2, m=7), dict(depth=0),
                dict(m=256), dict(V=64 * 8192 + 1),
                dict(k=16, depth=9, m=100), dict(k=16, depth=3, m=256), dict(B=-1)):
        assert sv.sv_eagle2_state_bytes(_e2(**bad)) == 0, bad
        assert sv.sv_last_error()


def test_eagle2_entry_points_reject_bad_host_arguments():
    c = _e2()
    need = sv.sv_eagle2_state_bytes(c)
    L = sv.lib()
    fake = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100004)
    # state: NULL, too small, misaligned
    assert L.sv_eagle2_begin(ctypes.byref(c), None, need, fake, None) == sv.SV_E_NULL
    assert L.sv_eagle2_begin(ctypes.byref(c), fake, need - 1, fake, None) == sv.SV_E_WORKSPACE
    assert L.sv_eagle2_begin(ctypes.byref(c), ctypes.c_void_p(0x100010), need, fake, None) == sv.SV_E_WORKSPACE
    assert L.sv_eagle2_begin(ctypes.byref(c), fake, need, None, None) == sv.SV_E_NULL
    # expand: step range, q NULL / misaligned
    assert L.sv_eagle2_expand(ctypes.byref(c), fake, need, -1, fake, None, None, None) == sv.SV_E_SHAPE
    assert L.sv_eagle2_expand(ctypes.byref(c), fake, need, 6, fake, None, None, None) == sv.SV_E_SHAPE
    assert L.sv_eagle2_expand(ctypes.byref(c), fake, need, 0, None, None, None, None) == sv.SV_E_NULL
    assert L.sv_eagle2_expand(ctypes.byref(c), fake, need, 0, odd, None, None, None) == sv.SV_E_UNSUPPORTED
    # finish: every output is required
    assert L.sv_eagle2_finish(ctypes.byref(c), fake, need, fake, fake, fake, fake, None, None) == sv.SV_E_NULL
    # expand + finish: the checks of both
    assert L.sv_eagle2_expand_finish(ctypes.byref(c), fake, need, 6, fake, fake, fake, fake, fake, fake,
                                     None) == sv.SV_E_SHAPE
    assert L.sv_eagle2_expand_finish(ctypes.byref(c), fake, need, 5, None, fake, fake, fake, fake, fake,
                                     None) == sv.SV_E_NULL
    assert L.sv_eagle2_expand_finish(ctypes.byref(c), fake, need, 5, odd, fake, fake, fake, fake, fake,
                                     None) == sv.SV_E_UNSUPPORTED
    assert L.sv_eagle2_expand_finish(ctypes.byref(c), fake, need, 5, fake, fake, None, fake, fake, fake,
                                     None) == sv.SV_E_NULL
    assert L.sv_eagle2_expand_finish(ctypes.byref(c), fake, need - 1, 5, fake, fake, fake, fake, fake, fake,
                                     None) == sv.SV_E_WORKSPACE
    bad = _e2(k=0)
    assert L.sv_eagle2_finish(ctypes.byref(bad), fake, need, fake, fake, fake, fake, fake, None) == sv.SV_E_SHAPE
    # B = 0: nothing to do, no pointer is looked at
    z = _e2(B=0)
    assert L.sv_eagle2_begin(ctypes.byref(z), None, 0, None, None) == sv.SV_OK


def test_plain_c_client_builds_and_passes(tmp_path):
    """The header and library serve a C program directly: gcc compiles a
    client against include/sv.h, links libsv.so, and runs its host checks."""
    src = os.path.join(ROOT, "tests", "abi_host_check.c")
    exe = str(tmp_path / "abi_host_check")
    libdir = os.path.dirname(sv.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                        "-L", libdir, "-lsv", "-Wl,-rpath," + libdir, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed" in r.stdout


def test_draft_head_host_checks():
    L = sv.lib()
    fake = 0x100000

    def args(**kw):
        a = sv.SvHeadArgs(8, 8192, 256, 128256, 256, 2, fake, fake, fake, fake, fake, fake, fake, fake)
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    assert L.sv_draft_head(None, None) == sv.SV_E_NULL
    for bad, code in ((dict(d=100), sv.SV_E_SHAPE), (dict(r=48), sv.SV_E_SHAPE), (dict(n=0), sv.SV_E_SHAPE),
                      (dict(N=-1), sv.SV_E_SHAPE), (dict(tile=24), sv.SV_E_UNSUPPORTED),
                      (dict(tile=512), sv.SV_E_UNSUPPORTED), (dict(k_tile=9), sv.SV_E_UNSUPPORTED),
                      (dict(k_tile=0), sv.SV_E_UNSUPPORTED), (dict(r=4096), sv.SV_E_UNSUPPORTED),
                      (dict(W=None), sv.SV_E_NULL), (dict(h=fake + 8), sv.SV_E_UNSUPPORTED)):
        a = args(**bad)
        assert L.sv_draft_head(ctypes.byref(a), None) == code, bad
        assert sv.sv_last_error()
    assert L.sv_draft_head(ctypes.byref(args(N=0, h=None, W=None)), None) == sv.SV_OK
