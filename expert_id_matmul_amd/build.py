"""Build libeidm.so (all HIP sources, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libeidm.so")
SOURCES = ["eidm_api.hip", "route.hip", "map.hip", "matmul_direct.hip", "matmul_grouped.hip",
           "combine.hip", "moe_direct.hip", "validate.hip", "calibrate.hip", "ffn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep packed-f32 VALU forms out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no contraction or fast-math: every fma is written out; f32 divide correctly rounded
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if out.strip() and verbose:
        print(out)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
