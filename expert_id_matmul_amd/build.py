"""Build libeidm.so (all HIP sources, gfx950) in-tree with hipcc: one object
per source, compiled in parallel, then one link."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libeidm.so")
OBJ = os.path.join(PKG, "_build")
SOURCES = ["eidm_api.hip", "route.hip", "map.hip", "matmul_direct.hip", "matmul_grouped.hip",
           "matmul_grouped16.hip", "combine.hip", "moe_direct.hip", "validate.hip", "calibrate.hip",
           "ffn.hip", "noalloc.hip", "matmul_split16.hip", "matmul_grouped16_acc.hip"]
# per-source extra flags: the long-job build of the 16x16x1 Grouped kernel
# keeps its matrix-core accumulators in the architectural registers (the
# slice sums are then read by ordinary adds, with no accumulator-register
# moves); matmul_grouped16_acc.hip, the short-job build, keeps the default
EXTRA = {"matmul_grouped16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep packed-f32 VALU forms out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no contraction or fast-math: every fma is written out; f32 divide correctly rounded
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _filter(text: str) -> str:
    return "\n".join(line for line in text.splitlines() if "packed-fp32-ops" not in line)


def _compile(src: str, verbose: bool) -> tuple[str, str]:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", obj + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = _filter(proc.stdout + proc.stderr)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({proc.returncode}):\n{out}")
    os.replace(obj + ".tmp", obj)
    return obj, out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    for _, out in results:
        if out.strip() and verbose:
            print(out)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in results], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed ({proc.returncode}):\n{_filter(proc.stdout + proc.stderr)}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
