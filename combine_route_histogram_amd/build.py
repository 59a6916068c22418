"""Build libmdc.so (HIP, gfx950) in-tree: python combine_route_histogram_amd/build.py

Run it as a script (or load it by path): importing the package needs the built library.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# kernel sources compiled into the one library; mdc_common.h is shared by both
SRCS = [os.path.join(PKG, "csrc", "mdc_dispatch.hip"), os.path.join(PKG, "csrc", "mdc_ffn.hip")]
INC = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmdc.so")
# the memory-ceiling probes the benchmark times beside the library (a library of their own)
PROBE_SRCS = [os.path.join(PKG, "csrc", "mdc_probe.hip")]
PROBE_OUT = os.path.join(PKG, "libmdc_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # fp32 products and sums of the combine are rounded one by one (no FMA contraction)
    "-ffp-contract=off",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _build_one(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libmdc.so and libmdc_probe.so (always, also where they exist)."""
    _build_one(PROBE_SRCS, PROBE_OUT, verbose)
    return _build_one(SRCS, OUT, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
