"""Build ``lib/libzero_flat.so`` for gfx950 with hipcc.

Usage: ``python -m zero_sharded_mixed_flat_amd.build`` (or ``build()``).  Always
recompiles.  The host partitioner is plain C++; the kernels are HIP for gfx950
only.  Packed fp32 instructions are disabled on the device side.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libzero_flat.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _cxx():
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler found")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose=True):
    hipcc = _hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]
    # The partitioner is plain host C++.
    plan_o = os.path.join(objdir, "plan.o")
    _run([_cxx(), *common, "-c", os.path.join(CSRC, "plan.cpp"), "-o", plan_o])
    objs = [plan_o]
    # Host AdamW (host code only, built by the host compiler): IEEE fp64 with no
    # contraction, so every instruction set gives the same bits.
    host_flags = [f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__"]
    offload_o = os.path.join(objdir, "offload.o")
    _run([_cxx(), *common, "-ffp-contract=off", *host_flags, "-c", os.path.join(CSRC, "offload.cpp"),
          "-o", offload_o])
    ckpt_o = os.path.join(objdir, "ckpt.o")
    _run([_cxx(), *common, *host_flags, "-c", os.path.join(CSRC, "ckpt.cpp"), "-o", ckpt_o])
    objs += [offload_o, ckpt_o]
    for src in ("kernels.hip", "quant.hip"):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        _run([hipcc, *common, "-x", "hip", f"--offload-arch={ARCH}",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
