"""Build the gfx950 HIP library libmxq.so in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("mxq.hip", "mxq_calib.hip", "mxq_gemm.hip", "mxq_norm.hip", "mxq_block.hip")]
LIBRARY = os.path.join(PKG, "libmxq.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxq.so)")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no packed-fp32 VALU ops (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels run with the IEEE mode bit clear: v_max/v_min need no
    # canonicalizing copies (NaN inputs are outside the contract)
    "-mno-amdgpu-ieee", "-fno-honor-nans",
    # matrix-core results straight into VGPRs (no accumulator copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def command(out: str = LIBRARY, defines=()) -> list[str]:
    return [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"),
            *[f"-D{d}" for d in defines], "-o", out, *SOURCES]


def build(out: str = LIBRARY, defines=()) -> str:
    tmp = out + ".tmp"
    subprocess.run(command(tmp, defines), check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
