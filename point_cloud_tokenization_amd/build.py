"""Build libfpstok.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfpstok.so")
SOURCES = [os.path.join(CSRC, "fpstok_kernels.hip"), os.path.join(CSRC, "fpstok_api.cpp")]
HEADERS = [os.path.join(ROOT, "include", "fpstok.h"), os.path.join(CSRC, "fpstok_internal.h")]

ARCH = "gfx950"
# -ffp-contract=off: the squared distance is the exact float32 sequence
#   ((dx*dx + dy*dy) + dz*dz) + dt*dt, never fused into FMAs.
# -packed-fp32-ops is switched off: hipcc must not form v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the register-resident FPS reads its pulse arrays with a uniform dynamic
    # index; this limit lets every instantiation keep them in VGPRs (no
    # scratch memory)
    "-mllvm", "-amdgpu-promote-alloca-to-vector-limit=1024",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP source for gfx950 into libfpstok.so (always rebuilds)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_path: str) -> str:
    """Compile the kernels to gfx950 assembly (for the build checks)."""
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")],
           "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", out_path, SOURCES[0]]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
