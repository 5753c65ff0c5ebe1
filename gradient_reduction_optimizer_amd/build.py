"""Build libgro.so (the C-ABI library) and libgro_probe.so (streaming
probes for the benchmark) in-tree for gfx950.

    python -m gradient_reduction_optimizer_amd.build
    python -m gradient_reduction_optimizer_amd.build --variant NAME [DEFINE=VALUE ...]

The planner is plain C++ (g++); the device entry points and kernels are HIP
(hipcc, gfx950 only).  No contraction of FP operations anywhere, so each
FP32 step rounds once; packed-FP32 instruction selection is switched off.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgro.so")
PROBE_LIB = os.path.join(PKG, "libgro_probe.so")
CLIENT = os.path.join(BUILD, "abi_client")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libgro.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    o = os.path.join(BUILD, "plan.o")
    _run(["g++", *COMMON, "-c", os.path.join(CSRC, "plan.cpp"), "-o", o], verbose)
    objs.append(o)
    for name in ("kernels", "abi"):
        o = os.path.join(BUILD, f"{name}.o")
        _run([HIPCC, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, f"{name}.hip"), "-o", o], verbose)
        objs.append(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # Streaming probes (measurement only; bench.py reports what the kernels'
    # access patterns can reach): a separate library, not part of the ABI.
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *COMMON, *HIP_FLAGS, "-shared", os.path.join(CSRC, "stream_probe.hip"), "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    # A plain C client of the ABI (used by the tests): C compiler, HIP
    # runtime headers and library, linked against libgro.so.
    client = os.path.join(ROOT, "tests", "native", "abi_client.c")
    if os.path.exists(client):
        _run(["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
              f"-I{ROCM}/include", client, "-o", CLIENT, f"-L{PKG}", "-lgro", f"-L{ROCM}/lib",
              "-lamdhip64", "-Wl,-rpath,$ORIGIN/..", f"-Wl,-rpath,{ROCM}/lib"], verbose)
    return LIB


VARIANTS = os.path.join(BUILD, "variants")


def build_variant(name: str, defines, verbose: bool = False) -> str:
    """Build libgro.so with compile-time knobs (e.g. ["GRO_UNROLL_WIN=4"]) as
    _build/variants/libgro_<name>.so, for launch-shape comparisons with
    `bench.py --lib`.  The in-tree libgro.so is not touched."""
    os.makedirs(VARIANTS, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    objs = []
    o = os.path.join(VARIANTS, f"{name}_plan.o")
    _run(["g++", *COMMON, *dflags, "-c", os.path.join(CSRC, "plan.cpp"), "-o", o], verbose)
    objs.append(o)
    for src in ("kernels", "abi"):
        o = os.path.join(VARIANTS, f"{name}_{src}.o")
        _run([HIPCC, *COMMON, *HIP_FLAGS, *dflags, "-c", os.path.join(CSRC, f"{src}.hip"), "-o", o], verbose)
        objs.append(o)
    out = os.path.join(VARIANTS, f"libgro_{name}.so")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out], verbose)
    for o in objs:
        os.remove(o)
    return out


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of the kernels (for inspection)."""
    _run([HIPCC, *COMMON, *HIP_FLAGS, "--cuda-device-only", "-S",
          os.path.join(CSRC, "kernels.hip"), "-o", out_path], False)
    return out_path


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "--variant":
        # python -m gradient_reduction_optimizer_amd.build --variant NAME [DEFINE=VALUE ...]
        print(build_variant(sys.argv[2], sys.argv[3:]))
    else:
        print(build(verbose="-v" in sys.argv))
