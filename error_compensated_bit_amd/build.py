"""Build the gfx950 shared library libecho_amd.so in-tree with hipcc.

Flags that matter for the results:
  -ffp-contract=off        no a*b+c is fused except the dequantizer's explicit fmaf
  -fhip-fp32-correctly-rounded-divide-sqrt
                           IEEE division (the quantizer step and its reciprocal)
  -target-feature -packed-fp32-ops
                           no packed fp32 instructions are generated
fp32 denormals are kept (no -fgpu-flush-denormals-to-zero).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("echo_api.hip", "echo_kernels.hip")]
HEADERS = [os.path.join(ROOT, "include", "echo.h"), os.path.join(CSRC, "echo_internal.h")]
ARCH = "gfx950"


def library_path() -> str:
    return os.path.join(HERE, "libecho_amd.so")


def hipcc_flags() -> list[str]:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    out = library_path()
    tmp = out + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc"] + hipcc_flags() + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
