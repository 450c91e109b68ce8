"""Compile the C test programs of tests/c_abi against include/fsdpshard.h and the built library.

    python tests/c_abi/build.py

host_check and host_edges need only the C library; gpu_step also links the HIP runtime.
Binaries go to tests/c_abi/bin/ and find libfsdpshard.so through an rpath relative to their own
location.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "fsdp_sharded_optimizer_layout_amd")
BIN = os.path.join(HERE, "bin")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

COMMON = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", f"-I{os.path.join(ROOT, 'include')}"]
# $ORIGIN-relative, so the binaries find the library wherever the repository is copied.
LINK = [f"-L{PKG}", "-lfsdpshard", "-Wl,-rpath,$ORIGIN/../../../fsdp_sharded_optimizer_layout_amd"]
# A plain C compiler must name the platform for the HIP runtime header (hipcc does it itself).
HIP = ["-D__HIP_PLATFORM_AMD__", f"-isystem{os.path.join(ROCM, 'include')}"]
HIP_LINK = [f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]


def commands():
    return [
        COMMON + [os.path.join(HERE, "host_check.c"), "-o", os.path.join(BIN, "host_check")] + LINK,
        COMMON + [os.path.join(HERE, "host_edges.c"), "-o", os.path.join(BIN, "host_edges")] + LINK,
        COMMON + HIP + [os.path.join(HERE, "gpu_step.c"), "-o", os.path.join(BIN, "gpu_step")]
        + LINK + HIP_LINK,
    ]


def build(verbose=False):
    os.makedirs(BIN, exist_ok=True)
    for cmd in commands():
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
