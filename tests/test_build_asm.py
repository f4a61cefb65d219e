"""Checks on the gfx950 assembly of the attention kernels (no GPU needed).

The attention kernels stage K/V tiles with global_load_lds_dwordx4 issued from
inline asm that first writes m0 (the LDS destination of the copy).  m0 is a
register the compiler reserves for itself: declaring it clobbered does not
make the compiler save a value of its own around the asm.  The copies are
therefore only safe while the compiler keeps nothing in m0 in these kernels.
This test compiles attn.hip with the library's own flags and checks, for
every kernel, that each access to m0 is one of the copy sequences: a scalar
move into m0 immediately followed by its global_load_lds.
"""
import os
import re
import shutil
import subprocess

import pytest

from eagle_tree_verification_attn_amd import build as svbuild

SRC = os.path.join(svbuild.CSRC, "attn.hip")


def _device_asm(tmp_path):
    out = str(tmp_path / "attn.s")
    cmd = [svbuild.HIPCC, *[f for f in svbuild.CFLAGS if f not in ("-fPIC",) and not f.startswith("--offload-arch")],
           f"--offload-arch={svbuild.ARCH}", *svbuild.FILE_FLAGS.get("attn.hip", []),
           "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().split("\n")


def _kernels(lines):
    """(name, instruction lines) of every kernel in the listing."""
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN2sv\S*:", l)]
    for i in starts:
        name = lines[i].split(":")[0]
        end = next(j for j in range(i, len(lines)) if ".Lfunc_end" in lines[j])
        body = [l.strip() for l in lines[i + 1:end]]
        yield name, [l for l in body if l and not l.startswith(";") and not l.startswith(".")]


@pytest.mark.skipif(not os.path.exists(svbuild.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_m0_only_in_the_copy_sequences(tmp_path):
    lines = _device_asm(tmp_path)
    kernels = list(_kernels(lines))
    assert any("k_attn_bf16" in n for n, _ in kernels)
    copies = 0
    for name, ins in kernels:
        for k, l in enumerate(ins):
            if not re.search(r"\bm0\b", l):
                continue
            ok = l.startswith("s_mov_b32 m0, s") and k + 1 < len(ins) and ins[k + 1].startswith("global_load_lds_dwordx4")
            assert ok, f"{name}: m0 used outside a copy sequence: {l!r}"
            copies += 1
    assert copies > 0
