"""Build the HIP library ``libnf4bwd.so`` in-tree with hipcc for gfx950.

Usage: ``python dequant_backward_gemm_amd/build.py`` (or ``build()`` loaded from
this file).  It does not import the package, which loads the library at
import time.  Every call compiles from source.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libnf4bwd.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["nf4_abi.hip", "nf4_plan.hip", "nf4_dequant.hip", "nf4_pack.hip", "nf4_grad_a.hip",
           "nf4_grad_a_wide.hip", "nf4_grad_a_skinny.hip", "nf4_forward.hip", "nf4_forward_skinny.hip", "rms_norm_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # fp32 denormals kept (IEEE), no fast-math: the decode multiply and the
    # fp16 conversions must be the IEEE operations.
    "-fno-gpu-flush-denormals-to-zero",
    # LDS buffers are viewed with several element types
    "-fno-strict-aliasing",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the NF4 library)")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile all HIP sources into the in-tree shared library; return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
