"""Build libep.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

    python -m combine_get_dispatch_amd.build

Flags:
  --offload-arch=gfx950            CDNA4 only; no other target, no CUDA path
  -O3 -std=c++17 -fPIC -shared
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                   keep the compiler from forming packed fp32
                                   (v_pk_*_f32) instructions
  -fhip-fp32-correctly-rounded-divide-sqrt
                                   IEEE fp32 division for the FP8 scales
  -fno-gpu-flush-denormals-to-zero fp32 denormals kept (the FP8 products and
                                   the fp32 sums are exact IEEE operations)
  -ffp-contract=off                only the explicit fmaf() calls are fused
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libep.so")
SOURCES = [os.path.join(CSRC, "ep_kernels.hip"), os.path.join(CSRC, "ep_api.hip"), os.path.join(CSRC, "ep_patterns.hip")]
HEADERS = [os.path.join(CSRC, "ep_internal.h"), os.path.join(INCLUDE, "ep.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libep.so)")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
            "-ffp-contract=off", "-Wall", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source (always; this is the does-it-build check)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + ["-shared", "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
