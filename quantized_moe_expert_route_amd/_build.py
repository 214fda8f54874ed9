"""Build the HIP library (libmoe_route.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_route.so")
SOURCES = ["moe_kernels.hip", "moe_grouped.hip", "moe_mx.hip", "moe_probe.hip", "moe_api.cpp",
           "moe_pool.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-fast-math",
    "-ffp-contract=fast",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fvisibility=hidden",
    # never emit packed fp32 math (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs (no accumulator-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, jobs: int = 2) -> str:
    cc = hipcc()
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-x")
            cmd.insert(2, "hip")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    for p, cmd in procs:
        if p.wait() != 0:
            raise RuntimeError("compile failed: " + " ".join(cmd))
    tmp = LIB + ".tmp"
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
