"""Build the gfx950 HIP library libmxq.so in-tree with hipcc.

Each source is compiled to its own object (with the flags `flags_for`
gives it) and the objects are linked into one shared library."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCE_NAMES = ("mxq.hip", "mxq_calib.hip", "mxq_gemm.hip", "mxq_norm.hip", "mxq_block.hip")
SOURCES = [os.path.join(PKG, "csrc", f) for f in SOURCE_NAMES]
LIBRARY = os.path.join(PKG, "libmxq.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxq.so)")


VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no packed-fp32 VALU ops (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels run with the IEEE mode bit clear: v_max/v_min need no
    # canonicalizing copies (NaN inputs are outside the contract)
    "-mno-amdgpu-ieee", "-fno-honor-nans",
    # matrix-core results straight into VGPRs (no accumulator copies)
    *VGPR_FORM,
]
# Sources built without the VGPR form (a kernel that keeps more accumulator
# registers than the VGPR file holds needs them in AGPRs).  None at present.
NO_VGPR_FORM: set[str] = set()


def flags_for(source: str) -> list[str]:
    if os.path.basename(source) in NO_VGPR_FORM:
        return [f for f in FLAGS if f not in VGPR_FORM]
    return list(FLAGS)


def compile_command(source: str, obj: str, defines=()) -> list[str]:
    flags = [f for f in flags_for(source) if f != "-shared"]
    return [hipcc(), *flags, "-c", "-I", os.path.join(ROOT, "include"),
            *[f"-D{d}" for d in defines], "-o", obj, source]


def link_command(objs, out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs]


def command(out: str = LIBRARY, defines=()) -> list[list[str]]:
    """The compile commands (one per source) and the link command."""
    objs = [os.path.join(os.path.dirname(out), os.path.basename(s) + ".o") for s in SOURCES]
    return [compile_command(s, o, defines) for s, o in zip(SOURCES, objs)] + [link_command(objs, out)]


def build(out: str = LIBRARY, defines=()) -> str:
    with tempfile.TemporaryDirectory(prefix="mxq_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            futs = [ex.submit(subprocess.run, compile_command(s, o, defines), check=True)
                    for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        tmp_out = out + ".tmp"
        subprocess.run(link_command(objs, tmp_out), check=True)
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build())
