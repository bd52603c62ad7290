"""Build librlq.so (HIP, gfx950) in-tree with hipcc.

    python -m decode_attention_rlq_amd.build

The library lands next to this file; the Python binding loads it from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librlq.so")
SOURCES = ("rlq_host.hip", "rlq_append.hip", "rlq_decode.hip", "rlq_decode_wide.hip")

# Packed fp32 VALU ops are kept out of the generated code: hipcc would form
# them from ordinary float code, and the kernels do not need them.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librlq)")


# Microbenchmarks of the GPU's ceilings (HBM read stream, MFMA and LDS rates,
# shader clock) for bench.py's rooflines; not part of the decode path.
CEILINGS_SOURCES = ("rlq_ceilings.hip",)
CEILINGS_LIB = os.path.join(PKG, "librlq_ceilings.so")


def _compile(srcs, out, verbose, extra_flags=()):
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in srcs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    _compile(CEILINGS_SOURCES, CEILINGS_LIB, verbose)
    return _compile(SOURCES, LIB, verbose, extra_flags)


if __name__ == "__main__":
    print(build(verbose=True))
