"""Build the HIP verification library (libsv.so) for gfx950, in place.

    python -m eagle_tree_verification_attn_amd.build

Every source under csrc/ is compiled by hipcc for gfx950 and linked into
eagle_tree_verification_attn_amd/libsv.so next to this file.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsv.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("SV_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Per-file flags.  attn.hip: scores are finite or -inf (masked), never NaN by
# construction of the kernel, so max needs no NaN canonicalisation; the
# scheduler's AMDGPU register-pressure trackers give the attention kernels a
# schedule measured about 2% faster on gfx950, with the same registers and
# bit-identical results.
FILE_FLAGS = {"attn.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-use-amdgpu-trackers=1"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in l and l.strip()]
    return obj, r.returncode, "\n".join(msgs), cmd


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    failed = False
    for obj, rc, msg, cmd in results:
        if msg and (verbose or rc):
            print(msg, file=sys.stderr)
        if rc:
            print("FAILED: " + " ".join(cmd), file=sys.stderr)
            failed = True
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[r[0] for r in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(r.stdout + r.stderr, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
