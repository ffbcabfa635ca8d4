"""Build ``libbsgemm.so`` (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Usage: ``python -m mx_grouped_gemm_amd.build`` (or ``build()`` from Python). Always
recompiles. Object files go to ``_build/`` at the repository root; the shared library is
written next to this file.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libbsgemm.so")

SOURCES = ["bsgemm_api.cpp", "tile_map.hip", "bs_fp8_grouped.hip", "mx_scaled.hip", "permute.hip", "bs_fp8_small_m.hip",
           "nv_fp4.hip"]

# -packed-fp32-ops off: no packed fp32 VALU instructions are generated.
# -amdgpu-mfma-vgpr-form: MFMA results go to VGPRs, so the promote FMAs read them directly
#   instead of copying them out of AGPRs first. Not for the nvfp4 kernel: no VALU reads its
#   accumulators inside the K loop, and they need the AGPRs (256 per lane, one wave per SIMD).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACC_SOURCES = {"nv_fp4.hip"}


def _hipcc():
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found (looked for {cand})")
    return cand


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless
    noise = "is not a recognized feature for this target"
    text = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{text}")
    return text


def build(verbose=False):
    """Compile every HIP source for gfx950 and link ``libbsgemm.so``. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        # a loop the source requires unrolled (#pragma clang loop unroll(full)) that the compiler
        # cannot unroll is a build error
        extra = ["-Werror=pass-failed"] if src in AGPR_ACC_SOURCES else VGPR_FORM
        cmds.append([hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
