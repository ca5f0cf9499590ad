"""Builds libpisa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_sparse_attention_stats_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpisa.so")
SOURCES = ["k_stats.hip", "k_select.hip", "k_fwd.hip", "pisa_abi.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no packed-fp32 VALU forms in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_abi", "pisa_c_caller.c")
C_CALLER = os.path.join(ROOT, "tests", "c_abi", "pisa_c_caller")


def build_c_caller(verbose: bool = False) -> str:
    """The plain C caller of the ABI (a test fixture): gcc, C99, linked to the
    in-tree libpisa.so and the HIP runtime."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(rocm, "include"), "-I" + os.path.join(ROOT, "include"),
           C_CALLER_SRC, "-o", C_CALLER, "-L" + PKG, "-lpisa", "-L" + os.path.join(rocm, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../block_sparse_attention_stats_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for the C caller:\n{r.stderr}")
    if verbose:
        print("built", C_CALLER)
    return C_CALLER


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_c_caller(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
