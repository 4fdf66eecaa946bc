"""Build libswa.so (HIP, gfx950) in-tree with hipcc.

    python -m sliding_window_attention_swa_amd.build

Compiles every source under csrc/ to an object (in parallel) and links them
into sliding_window_attention_swa_amd/libswa.so.  Always recompiles.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libswa.so")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", INCLUDE, "-I", CSRC,
    # Packed fp32 VALU ops stay off: all fp32 math is emitted as scalar-lane ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # No implicit fma contraction: only explicit fmaf() fuses, so every
    # instantiation of a kernel (e.g. f32 and bf16 output) computes the same
    # f32 values and the bf16 output is exactly the f32 output rounded.
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]
SOURCES = ["api.cpp", "index_kernels.hip", "store_kernels.hip", "decode_kernels.hip", "extend_kernels.hip",
           "validate_kernels.hip", "evict_kernels.hip", "alloc_kernels.hip", "probe_kernels.hip"]
# Per-source extra flags.  The MFMA probe's accumulators stay in VGPRs: in the
# AGPR form the compiler rotates the loop-carried accumulators through
# v_accvgpr moves every iteration, and the probe would time those moves.
EXTRA = {"probe_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libswa")
    return path


def _compile(src: str) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *lang, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in line)  # host pass does not know the GPU feature
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile and link libswa.so; returns its path."""
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
