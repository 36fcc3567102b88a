"""Build libtiledattn.so in-tree with hipcc for gfx950.

    python -m tiled_attention_09_amd.build        # or __graft_entry__.build()

Always recompiles.  The kernel resource report (VGPR/AGPR/SGPR, LDS, spills,
occupancy) from ``-Rpass-analysis=kernel-resource-usage`` is written to
``_build/resource_usage.txt`` (not committed).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("attn_fwd.hip", "attn_bwd.hip", "attn_fp8.hip")]
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libtiledattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

# Packed fp32 VALU forms are kept off: the compiler would otherwise fuse
# pairs of fp32 multiplies into them.
# The kernels take no NaN inputs (finite Q, K, V is a documented precondition;
# masking uses -inf, never NaN), which lets max chains fuse into v_max3.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans",
               "-Rpass-analysis=kernel-resource-usage"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_library(extra_flags=(), verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = OUT + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + ["-I", INCLUDE] + SRCS + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    report = os.path.join(BUILD_DIR, "resource_usage.txt")
    with open(report, "w") as f:
        f.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (%d); see %s" % (res.returncode, report))
    # Every kernel must have its host launch stub defined: clang can drop one
    # silently when a host-side check of the kernel body fails.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "__device_stub__" in ln]
    if nm.returncode != 0 or missing:
        raise RuntimeError("built library has undefined kernel stubs: %s" % missing)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build_library(sys.argv[1:], verbose=True)
