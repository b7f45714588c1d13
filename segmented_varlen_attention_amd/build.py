"""Build libgvattn.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m segmented_varlen_attention_amd.build`` (or call
``build()``).  Sources are compiled in parallel into ``_build/`` at the
repository root and linked into ``segmented_varlen_attention_amd/libgvattn.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libgvattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = os.environ.get("GVATTN_ARCH", "gfx950")

SOURCES = [
    "gvattn_api.hip",
    "gvattn_plan.hip",
    "gvattn_fwd_mfma.hip",
    "gvattn_fwd_fp32.hip",
    "gvattn_merge.hip",
    "gvattn_bwd.hip",
]

# Packed FP32 VALU ops are kept out of the generated code; the host pass
# warns that it does not know the feature, which is harmless.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions.  The forward's d > 128 kernels run one wave per SIMD
# with up to 512 registers; by default their MFMAs would accumulate in AGPRs
# and every vector operation on O or the scores would copy them to VGPRs and
# back.  The VGPR form keeps O and the scores in VGPRs (the Q fragments,
# only ever a matrix-core operand, are placed in AGPRs by the kernel).
# Kernels with at most 256 registers per wave use the VGPR form anyway.
SOURCE_FLAGS = {
    "gvattn_fwd_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgvattn)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link libgvattn.so.  Always
    recompiles.  Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
    jobs = jobs or min(len(cmds), 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
