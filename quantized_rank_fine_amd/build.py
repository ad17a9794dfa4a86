"""Build libqlora.so (HIP, gfx950) in-tree.

Compiles every source under ``csrc/`` with hipcc into ``_build/`` (parallel
object builds) and links ``quantized_rank_fine_amd/libqlora.so``.  Always
rebuilds; nothing is cached between calls.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlora.so")

SOURCES = ["api.cpp", "tables.cpp", "quantize.hip", "skinny.hip", "gemm.hip", "smallm.hip",
           "merge.hip", "optim.hip", "loftq.hip", "loftq.cpp", "noalloc.hip"]

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]
DEVICE = [
    f"--offload-arch={ARCH}",
    # keep packed fp32 ALU ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source device flags.  The skinny kernels keep their few MFMA
# accumulators in the VGPR file (no AGPR<->VGPR copies of loop-carried
# accumulators); the fused GEMMs hold 256 accumulator registers per lane and
# need the AGPR file for them.
DEVICE_EXTRA = {
    "skinny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "quantize.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "smallm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE + DEVICE_EXTRA.get(src, [])
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (o, err) in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
