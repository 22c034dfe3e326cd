"""Builds libdita.so in-tree with hipcc for gfx950.

    python partial_state_reuse_amd/build.py

(Run by path, not as a submodule: importing the package loads the library being rebuilt.)

Every HIP translation unit is compiled with packed-FP32 instructions disabled."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdita.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# MFMA results in VGPRs: the softmax and the rescales touch the accumulators with VALU ops,
# which cannot read AGPRs, so AGPR-resident accumulators cost a copy per element per use.
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose_resources: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    host_obj = os.path.join(build_dir, "dita_host.o")
    _run([HIPCC, "-std=c++17", "-O2", "-fPIC", "-Wall", "-c",
          os.path.join(CSRC, "dita_host.cpp"), "-o", host_obj] + inc)
    objs.append(host_obj)
    kern_obj = os.path.join(build_dir, "dita_kernels.o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if verbose_resources else []
    _run([HIPCC, "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-c",
          os.path.join(CSRC, "dita_kernels.hip"), "-o", kern_obj] + NO_PACKED_FP32 + MFMA_VGPR + inc
         + extra)
    objs.append(kern_obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose_resources="-v" in sys.argv)
