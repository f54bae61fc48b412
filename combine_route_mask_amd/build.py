"""Build the gfx950 HIP libraries in-tree with hipcc: ``libmoe_ep.so`` (the
exchange behind include/moe_ep.h) and ``libmoe_ep_ceilings.so`` (the
benchmark's plain reference kernels); then, with the host C compiler, the
plain C example that uses the exchange through its C ABI only
(``_build/moe_ep_example``)."""
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
# a C99 program over the C ABI alone (host code; links libmoe_ep.so and the HIP runtime)
EXAMPLE_SOURCE = os.path.join(HERE, "examples", "moe_ep_example.c")
EXAMPLE = os.path.join(HERE, "_build", "moe_ep_example")

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


def rocm_path() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def build_example(verbose: bool = False, out: str = EXAMPLE) -> str:
    """Compile the C example as C99 against include/moe_ep.h, linked to the
    in-tree libmoe_ep.so (found through its rpath) and the HIP runtime."""
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no host C compiler found for the C example")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    rocm = rocm_path()
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), "-o", tmp, EXAMPLE_SOURCE,
           "-L", HERE, "-lmoe_ep", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/..:" + HERE, "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("C example build failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile the exchange library libmoe_ep.so, the benchmark's
    reference-kernel library libmoe_ep_ceilings.so and the C example
    (always rebuilds)."""
    _compile(CEILINGS_LIB, CEILINGS_SOURCES, verbose)
    lib = _compile(LIB, SOURCES, verbose)
    build_example(verbose)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
