"""Builds libnsa_sel.so (HIP, gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "nsa_sel.hip")
LIB = os.path.join(PKG, "libnsa_sel.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep the compiler from forming packed fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax and the V^T conversion consume them
    # on the VALU, so AGPR destinations would only add copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(extra_flags=(), out: str = LIB, src: str = SRC) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-o", tmp, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
