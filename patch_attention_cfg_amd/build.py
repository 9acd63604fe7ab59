"""Build libdfp.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage:  python -m patch_attention_cfg_amd.build      (or build_library())
The library lands next to this file; objects go to <repo>/_build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdfp.so")

SOURCES = ["host.cpp", "kv_scatter.hip", "cfg_step.hip", "attention.hip", "attention_bf16.hip",
           "group_norm.hip"]

ARCH = "gfx950"
# Packed-FP32 VALU instructions are kept out of the device code on purpose.
# MFMA results go to ordinary VGPRs: a kernel whose LDS allows one
# workgroup per CU (the two-key-group attention) otherwise gets a
# 512-register budget, and the allocator then places MFMA results in AGPRs
# and copies them to VGPRs for the softmax every step (about 100 extra
# moves per step).  Kernels that fit 256 registers compile identically.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-command-line-argument"] + DEVICE_FLAGS


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    workers = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


C_CALLER_SRC = os.path.join(ROOT, "tests", "c", "step_from_c.c")
C_CALLER = os.path.join(ROOT, "tests", "c", "step_from_c")


def build_c_caller(verbose: bool = False) -> str:
    """The plain-C caller the tests run (host code only: gcc, the HIP runtime
    and libdfp.so)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = C_CALLER + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_CALLER_SRC, "-o", tmp,
           "-L", PKG, "-l:libdfp.so", "-Wl,-rpath,$ORIGIN/../../patch_attention_cfg_amd",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {C_CALLER_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, C_CALLER)
    if verbose:
        print("built", C_CALLER)
    return C_CALLER


if __name__ == "__main__":
    build_library(verbose=True)
    build_c_caller(verbose=True)
    sys.exit(0)
