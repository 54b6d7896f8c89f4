"""Build liblw.so (the HIP kernels for gfx950 plus the host bundle builder).

    python -m decode_gemv_amd.build

hipcc compiles each HIP source for gfx950 only; the host builder is plain
C++17.  Packed fp32 VALU forms are disabled on the device side.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblw.so")
ARCH = "gfx950"

HIP_SOURCES = ["runtime.hip", "fused_q.hip", "bf16.hip", "mfma.hip", "twin.hip", "mlp.hip", "skip.hip", "probe.hip", "rans.hip", "recon.hip"]
CXX_SOURCES = ["bundle.cpp"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build liblw")


def _common():
    return ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _hip_cmd(src, obj):
    return [hipcc(), "-c", "-x", "hip", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-munsafe-fp-atomics", *_common(), "-o", obj, src]


def _cxx_cmd(src, obj):
    return [hipcc(), "-c", "-x", "c++", *_common(), "-o", obj, src]


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append(_hip_cmd(os.path.join(CSRC, s), o))
        objs.append(o)
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append(_cxx_cmd(os.path.join(CSRC, s), o))
        objs.append(o)

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("compile failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
        return r.stderr

    with cf.ThreadPoolExecutor(jobs) as ex:
        for err in ex.map(run, cmds):
            if verbose and err.strip():
                print(err)
    tmp = LIB + ".tmp"
    run([hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs, "-L/opt/rocm/lib", "-lrocblas"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
