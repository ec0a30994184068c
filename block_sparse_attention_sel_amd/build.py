"""Builds the HIP libraries (gfx950) in-tree with hipcc:

- libnsa_sel.so: the selection-attention forward (include/nsa_sel.h), its
  backward (include/nsa_sel_bwd.h), the top-k block selection that produces
  its index rows (include/nsa_topk.h) and the dense / sliding-window attention
  forward it is compared with (include/nsa_dense.h);
- libnsa_gather_probe.so: the gather-ceiling probe (include/nsa_gather_probe.h),
  a measurement aid that replays the forward kernel's block gathers.
"""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRC = os.path.join(CSRC, "nsa_sel.hip")
DENSE_SRC = os.path.join(CSRC, "nsa_dense.hip")
BWD_SRC = os.path.join(CSRC, "nsa_sel_bwd.hip")
TOPK_SRC = os.path.join(CSRC, "nsa_topk.hip")
LIB = os.path.join(PKG, "libnsa_sel.so")
PROBE_SRC = os.path.join(CSRC, "gather_probe.hip")
PROBE_LIB = os.path.join(PKG, "libnsa_gather_probe.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep the compiler from forming packed fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax and the V^T conversion consume them
    # on the VALU, so AGPR destinations would only add copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # No NaN is ever produced or tested for (masked scores are -inf, which
    # stays legal): lets fmaxf compile to a bare v_max without quieting its
    # inputs first.
    "-fno-honor-nans",
]


def build(extra_flags=(), out: str = LIB, srcs=(SRC, DENSE_SRC, BWD_SRC, TOPK_SRC)) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build_all() -> list[str]:
    return [build(), build(out=PROBE_LIB, srcs=(PROBE_SRC,))]


if __name__ == "__main__":
    for path in build_all():
        print(path)
