"""Build librosa.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m online_suffix_automaton_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librosa.so")
ARCH = os.environ.get("ROSA_OFFLOAD_ARCH", "gfx950")


def command(out: str = LIB) -> list[str]:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    return ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            # packed fp32 instructions are kept out of all device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            *srcs, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building librosa.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
