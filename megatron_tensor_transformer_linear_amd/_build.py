"""Build of the gfx950 HIP library ``libtp_shard.so`` (in-tree, next to this file).

Each ``csrc/*.hip`` source is compiled to an object with hipcc for gfx950 (in parallel),
then the objects are linked into one shared library.  The measurement library
``libtp_calib.so`` (``calib/*.hip``: the matrix-core rate calibration the bench reports
beside the GEMMs) is built the same way.  No GPU is needed: hipcc cross-compiles.
Packed-fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
from typing import List, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libtp_shard.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
CALIB_SRC = os.path.join(HERE, "calib")
CALIB_LIB_PATH = os.path.join(HERE, "libtp_calib.so")

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-inline-asm",
                "-I" + INCLUDE] + DEVICE_FLAGS


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# Per-source device flags.  The attention kernel holds no NaN (masked scores are -inf), so its
# max reductions skip NaN quieting, which lets them fold into three-operand maxes.
SOURCE_FLAGS = {"attention.hip": ["-fno-honor-nans"]}


def sources(folder: str = CSRC) -> List[str]:
    return sorted(glob.glob(os.path.join(folder, "*.hip")))


def _run(cmd: List[str]) -> None:
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")


def _build_one(srcs: List[str], lib_path: str, obj_dir: str, flags: List[str],
               jobs: Optional[int]) -> str:
    hipcc = hipcc_path()
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, os.cpu_count() or 1), 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [hipcc] + flags + SOURCE_FLAGS.get(os.path.basename(s), [])
                          + ["-c", s, "-o", o]) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = lib_path + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, lib_path)
    return lib_path


def build_library(jobs: Optional[int] = None, extra_flags: Optional[List[str]] = None) -> str:
    """Compile every source and link LIB_PATH, then the calibration library CALIB_LIB_PATH.
    Always recompiles.  Returns LIB_PATH."""
    flags = COMMON_FLAGS + list(extra_flags or [])
    _build_one(sources(), LIB_PATH, BUILD_DIR, flags, jobs)
    _build_one(sources(CALIB_SRC), CALIB_LIB_PATH, os.path.join(BUILD_DIR, "calib"), flags, jobs)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library())
