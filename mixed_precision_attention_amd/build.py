"""Builds libconfk.so (the decode step) and libconfk_probe.so (the
streaming-read probe, a measurement aid) for gfx950, in-tree, with hipcc.

Usage: python -m mixed_precision_attention_amd.build
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libconfk.so")
PROBE_LIB = os.path.join(HERE, "libconfk_probe.so")

SOURCES = ["abi.hip", "confidence.hip", "attention.hip", "ema_rank.hip", "compact.hip", "quantize.hip",
           "noalloc.hip"]
PROBE_SOURCES = ["probe.hip"]

# Packed fp32 VALU instructions are disabled: the compiler still vectorises
# fp16 work, and every fp32 op is a plain VOP.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _link(sources, out, verbose):
    srcs = [os.path.join(CSRC, x) for x in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _link(SOURCES, LIB, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
