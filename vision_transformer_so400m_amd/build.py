"""Build libsiglip.so (product) and libsiglip_test.so (the same library plus
the test hooks of include/siglip_test_hooks.h) in-tree with hipcc for gfx950.

Usage: python -m vision_transformer_so400m_amd.build   (or build() from Python)
Every call recompiles; objects go to _build/ next to the package. The kernels
are compiled once; only siglip.cpp is compiled a second time for the test
build, with SIGLIP_TEST_HOOKS defined.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsiglip.so")
OUT_TEST = os.path.join(PKG, "libsiglip_test.so")
BUILD_DIR = os.path.join(ROOT, "_build")
KERNEL_SOURCES = ["gemm.hip", "layernorm.hip", "attention.hip", "map.hip", "convert.hip"]
# (source, object name, extra flags): the library front end, product and test build
FRONT_ENDS = [("siglip.cpp", "siglip", []), ("siglip.cpp", "siglip_test", ["-DSIGLIP_TEST_HOOKS"])]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # packed FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-file additions. attention.hip (the encoder's attention kernels only; the
# MAP probe attention lives in map.hip): scores are never NaN (padded keys are
# -inf), so max needs no NaN canonicalisation of its operands.
FILE_FLAGS = {"attention.hip": ["-fno-honor-nans"]}


def _compile(job) -> str:
    src, name, extra = job
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, out)


def build(verbose: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(s, os.path.splitext(s)[0], []) for s in KERNEL_SOURCES] + FRONT_ENDS
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    kernels, product, test = objs[:len(KERNEL_SOURCES)], objs[-2], objs[-1]
    _link(kernels + [product], OUT)
    _link(kernels + [test], OUT_TEST)
    if verbose:
        print(f"built {OUT} and {OUT_TEST}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
