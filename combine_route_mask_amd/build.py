"""Build the gfx950 HIP libraries in-tree with hipcc: ``libmoe_ep.so`` (the
exchange behind include/moe_ep.h) and ``libmoe_ep_ceilings.so`` (the
benchmark's plain reference kernels)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_ep.so")
SOURCES = ["exchange.hip", "agrs.hip", "api.cpp"]
# reference kernels of the benchmark (measurement only; the exchange never calls them)
CEILINGS_LIB = os.path.join(HERE, "libmoe_ep_ceilings.so")
CEILINGS_SOURCES = ["ceilings.hip"]

# Packed-FP32 instructions are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe_ep.so)")


def _compile(out: str, sources, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in sources]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile the exchange library libmoe_ep.so and the benchmark's
    reference-kernel library libmoe_ep_ceilings.so (always rebuilds)."""
    _compile(CEILINGS_LIB, CEILINGS_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
