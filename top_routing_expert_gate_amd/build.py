"""Build libmoe.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m top_routing_expert_gate_amd.build

Compiles every ``csrc/*.hip`` with hipcc in parallel into ``_build/`` and
links ``top_routing_expert_gate_amd/libmoe.so``, plus ``libmoe_debug.so``
(the C ABI compiled with MOE_DEBUG_CHECKS).  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed-f32 VALU ops stay off: plain f32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


DEBUG_LIB = os.path.join(PKG, "libmoe_debug.so")


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", "_debug.o" if debug else ".o"))
    cmd = [hipcc(), *COMMON, *(["-DMOE_DEBUG_CHECKS"] if debug else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """libmoe.so, and libmoe_debug.so: the same objects except the C ABI,
    compiled with MOE_DEBUG_CHECKS (moe_dispatch checks its routing)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    abi = os.path.join(CSRC, "abi.hip")
    jobs = [(s, False) for s in srcs] + [(abi, True)]
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    release = objs[: len(srcs)]
    debug = [o for o, (s, _) in zip(release, jobs) if s != abi] + [objs[-1]]
    _link(release, LIB)
    _link(debug, DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
