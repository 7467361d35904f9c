"""Build libmoe.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m mixture_experts_layer_top_amd.build

Compiles every source under csrc/ with hipcc, in parallel, then links the
shared library next to this file.  Always recompiles (a build check must
not trust stale objects).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["moe_api.cpp", "route.hip", "permute.hip", "gemm.hip", "combine.hip",
           "gemm_bwd.hip", "backward.hip", "probe.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return h


def kernel_scratch(remarks: str) -> dict[str, int]:
    """Scratch (private) segment bytes per lane of every kernel, from hipcc's
    kernel-resource-usage remarks: {mangled name: bytes}."""
    out, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None:
            out[name] = int(m.group(1))
            name = None
    return out


def scratch_kernels(remarks: str) -> list[tuple[str, int]]:
    """Kernels with a scratch segment: (mangled name, bytes per lane)."""
    return [(n, b) for n, b in kernel_scratch(remarks).items() if b > 0]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # every kernel keeps its state in registers and LDS: a kernel that spills
    # (accumulators demoted to scratch run several times slower) is a build
    # error.  A kernel source whose remarks name no kernel would pass this
    # check without checking anything, so that is an error too.
    if src.endswith(".hip") and not kernel_scratch(r.stderr):
        raise RuntimeError(f"{src}: hipcc printed no kernel-resource-usage remarks; "
                           "the scratch check cannot run")
    spilled = scratch_kernels(r.stderr)
    if spilled:
        raise RuntimeError(f"{src}: kernels with scratch memory: {spilled}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
