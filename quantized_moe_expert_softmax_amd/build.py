"""Build the gfx950 HIP library (libmoe_mi355x.so) in-tree with hipcc.

Every source under csrc/ is compiled for --offload-arch=gfx950 (no other
target) into _build/, then linked into the package directory, where the
Python binding loads it.  Packed-FP32 instruction selection is disabled
(-packed-fp32-ops); FP32 atomics use the hardware instructions.

The library links the HIP runtime that PyTorch-ROCm ships (torch/lib,
found at build time, also put on the library's RUNPATH): one process must
not hold two HIP/HSA runtimes, and torch provides the device memory and
streams the library works on.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-mcode-object-version=5",
    "-I" + os.path.join(os.path.dirname(HERE), "include"),
]


# Per-file extra flags.  The expert GEMMs keep their MFMA accumulators in
# ordinary VGPRs: with the accumulation-register form the register allocator
# shuffles accumulators between register files on every K step.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"gemm_stream.hip": _VGPR_FORM, "gemm_tiled.hip": _VGPR_FORM}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is harmless
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def hip_runtime_dir() -> str:
    """Directory of the libamdhip64.so that torch loads."""
    import torch
    d = os.path.join(os.path.dirname(torch.__file__), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError("torch's libamdhip64.so not found under %s" % d)
    return d


def build(verbose: bool = False) -> str:
    """Compile and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    rt = hip_runtime_dir()
    cmd = ["g++", "-shared", "-fPIC", *objs, "-o", tmp, "-L" + rt, "-lamdhip64",
           "-Wl,-rpath," + rt, "-Wl,--no-undefined"]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError("link failed:\n" + proc.stdout)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
