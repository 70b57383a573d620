"""Builds libofa.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m persistent_transformer_train_amd.build   (or build() from Python)
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libofa.so")
ROOT = os.path.dirname(PKG)

SOURCES = ["ofa_kernels.hip", "ofa_host.cpp"]
HEADERS = ["ofa_types.h", "ofa_dev.h", "ofa_launch.h", "k_simple.h", "k_mfma.h", "k_attn.h", "k_decode.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions stay off (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, jobs: int = 2) -> str:
    """Compile every HIP source and link libofa.so.  Always recompiles."""
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        # the host pass does not know the packed-fp32 feature; that warning is noise
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
