"""Build libdsa.so (HIP, gfx950) in-tree with hipcc.

    python -m long_context_sparse_score_amd.build_lib [-v]

Every HIP source under csrc/ is compiled for gfx950 only.  Packed-FP32 VALU
instructions are switched off for device code.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
CSRC = os.path.join(_HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(_HERE, "libdsa.so")
CALIB_DIR = os.path.join(_HERE, "calib")
CALIB_PATH = os.path.join(_HERE, "libdsa_calib.so")  # bench-only calibration kernels
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file device flags.  The indexer's inputs are finite by contract, so its
# ReLU may skip the NaN-quieting pass fmaxf otherwise needs (one VALU op per
# head x key).
FILE_FLAGS = {
    "index_scores.hip": ["-fno-honor-nans"],
    "index_scores_fp8.hip": ["-fno-honor-nans"],
    "index_backward.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    objdir = os.path.join(_HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src,
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # The host pass does not know the packed-fp32 feature flag; that note is harmless.
        noise = "'-packed-fp32-ops' is not a recognized feature"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if err.strip() and verbose:
            print(err, flush=True)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    # The bench's calibration kernels: their own library, outside the C ABI.
    calib = sorted(glob.glob(os.path.join(CALIB_DIR, "*.hip")))
    tmp = CALIB_PATH + ".tmp"
    cmd = [HIPCC, *COMMON_FLAGS, "-shared", "-o", tmp, *calib]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on the calibration kernels:\n{r.stderr}")
    os.replace(tmp, CALIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
