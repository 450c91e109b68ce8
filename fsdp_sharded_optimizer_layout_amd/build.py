"""Build libfsdpshard.so in-tree with hipcc for gfx950 (MI355X).

    python -m fsdp_sharded_optimizer_layout_amd.build

Flags that matter for the results:
  -ffp-contract=off   every float32 multiply and add is rounded on its own (no fused multiply-add),
                      which is the arithmetic the step is defined with;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keep the compiler from emitting packed fp32 instructions;
  (default)           correctly rounded float32 division and square root, denormals kept.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfsdpshard.so")
ARCH = "gfx950"

HIP_SOURCES = [os.path.join(CSRC, "shard_step.hip"), os.path.join(CSRC, "reshard.hip"),
               os.path.join(CSRC, "calib.hip")]
HOST_SOURCES = [os.path.join(CSRC, "layout.cpp")]


def clang():
    for cand in (os.environ.get("HIP_CLANG"), "/opt/rocm/lib/llvm/bin/clang++",
                 shutil.which("amdclang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("ROCm clang++ not found (ROCm is required to build libfsdpshard.so)")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function"]
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _obj(objdir, src):
    return os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o")


def commands(out=LIB, objdir=None):
    objdir = objdir or os.path.join(PKG, "_build")
    cc = clang()
    cmds = [[cc, *COMMON, *HIP_FLAGS, f"-I{INCLUDE}", "-c", src, "-o", _obj(objdir, src)]
            for src in HIP_SOURCES]
    cmds += [[cc, *COMMON, f"-I{INCLUDE}", "-c", src, "-o", _obj(objdir, src)]
             for src in HOST_SOURCES]
    objs = [_obj(objdir, src) for src in HIP_SOURCES + HOST_SOURCES]
    cmds.append([cc, "--hip-link", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                 "-o", out])
    return objdir, cmds


def build(verbose=False):
    tmp = LIB + ".tmp"
    objdir, cmds = commands(tmp)
    os.makedirs(objdir, exist_ok=True)
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
