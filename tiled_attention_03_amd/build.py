"""Builds libta03.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m tiled_attention_03_amd.build`` (or ``build()``). Always
recompiles. Packed-f32 VALU instructions are disabled for every HIP source.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libta03.so")
PROBE_LIB = os.path.join(PKG, "libta03_probe.so")

SOURCES = ["ta03_api.cpp", "prefill.hip", "prefill16.hip", "decode.hip", "rope.hip",
           "backward.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-product results and accumulators in vector registers: left to
    # its heuristics, the compiler put some kernels' accumulators in the
    # accumulator file and copied them to vector registers and back around
    # every vector-ALU update (the online-softmax rescale, the decode's
    # softmax), which costs vector-ALU time the f32 products share.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libta03.so)")


def check_kernel_stubs(obj: str) -> None:
    """Fail when the host pass left a kernel's launch stub undefined (it can
    drop a kernel template's host side without a diagnostic); the library
    would then fail to load or launch."""
    nm = shutil.which("nm") or "/usr/bin/nm"
    out = subprocess.run([nm, obj], check=True, capture_output=True, text=True).stdout
    missing = [line.split()[-1] for line in out.splitlines()
               if "__device_stub__" in line and line.split()[0] == "U"]
    if missing:
        raise RuntimeError(f"{os.path.basename(obj)}: host pass dropped kernel stubs: {missing}")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *HIP_FLAGS, *lang, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        check_kernel_stubs(obj)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    # The benchmark's probes (the decode's read ceiling, the matrix / vector
    # ALU issue overlap): a separate library on top of libta03.so (the read
    # probe uses the decode's launch plan), never loaded by the product path.
    probe_objs = []
    for src in ("probe_decode_read.hip", "probe_mfma_valu.hip"):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        check_kernel_stubs(obj)
        probe_objs.append(obj)
    tmp = PROBE_LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *probe_objs, "-L", PKG, "-lta03",
           "-Wl,-rpath,$ORIGIN", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
