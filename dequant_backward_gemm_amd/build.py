"""Build the HIP library ``libnf4bwd.so`` in-tree with hipcc for gfx950.

Usage: ``python dequant_backward_gemm_amd/build.py`` (or ``build()`` loaded from
this file).  It does not import the package, which loads the library at
import time.  Every call compiles from source: each source file to an object
(in parallel), then one link.

``build(variant="barriers")`` builds ``libnf4bwd_barriers.so`` from the same
sources with ``NF4_EXTRA_BARRIERS`` defined: every kernel then separates each
of its LDS phases with an extra barrier (a workgroup barrier where all waves
take the same path, a wave-level drain where a wave works on its own LDS
area).  Its results must equal the release library's bit for bit: a missing
barrier in the release kernels (an LDS race) would show as a difference.
"""

from __future__ import annotations

import concurrent.futures
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
BARRIER_LIB_PATH = os.path.join(PKG_DIR, "libnf4bwd_barriers.so")
OBJ_DIR = os.path.join(PKG_DIR, "_build")

SOURCES = ["nf4_abi.hip", "nf4_plan.hip", "nf4_dequant.hip", "nf4_pack.hip", "nf4_grad_a.hip",
           "nf4_grad_a_wide.hip", "nf4_grad_a_skinny.hip", "nf4_grad_a_lines.hip", "nf4_forward.hip", "nf4_forward_skinny.hip", "rms_norm_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # fp32 denormals kept (IEEE), no fast-math: the decode multiply and the
    # fp16 conversions must be the IEEE operations.
    "-fno-gpu-flush-denormals-to-zero",
    # LDS buffers are viewed with several element types
    "-fno-strict-aliasing",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

VARIANTS = {"release": (LIB_PATH, []), "barriers": (BARRIER_LIB_PATH, ["-DNF4_EXTRA_BARRIERS=1"])}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the NF4 library)")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[-3:])}")


def build(verbose: bool = False, extra_flags: list[str] | None = None, variant: str = "release",
          jobs: int | None = None) -> str:
    """Compile all HIP sources into the in-tree shared library of `variant`; return its path."""
    out_path, vflags = VARIANTS[variant]
    flags = [*HIPCC_FLAGS, *vflags, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC]
    obj_dir = os.path.join(OBJ_DIR, variant)
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc(), *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    workers = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out_path + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    args = sys.argv[1:]
    for v in (args or ["release"]):
        print(build(verbose=True, variant=v))
