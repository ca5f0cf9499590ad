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
SOURCES = ["k_stats.hip", "k_mnorm.hip", "k_select.hip", "k_fwd.hip", "k_bwd.hip", "pisa_abi.hip"]
# Translation units: (source, object name, extra flags). k_fwd.hip is built
# twice: once for the bf16 fused pass and dense baseline with every MFMA result
# in VGPRs (its weights then read the score accumulators without a move), once
# the usual way for the rest (fp32, the per-block first-order variant). The
# backward kernels are built with MFMA results in VGPRs too: k_bwd_dq then
# keeps two tiles of rows in flight at two wavefronts per SIMD.
VGPR_FORM = ["-mllvm", "--amdgpu-mfma-vgpr-form=1"]
UNITS = [(src, src + ".o", VGPR_FORM if src == "k_bwd.hip" else []) for src in SOURCES] + [
    ("k_fwd.hip", "k_fwd_bf16.hip.o",
     ["-DPISA_FWD_VGPR_FORM=1", *VGPR_FORM]),
]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no packed-fp32 VALU forms in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(unit) -> str:
    src, obj, extra = unit
    out = os.path.join(OBJ, obj)
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


SAN_LIB = os.path.join(OBJ, "san", "libpisa_san.so")
# host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
# (the device code is built as usual: sanitizers apply to the host pass only)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build_host_sanitized(objs, verbose: bool = False) -> str:
    """A copy of the library whose ABI layer (argument validation, workspace
    layout, launch order: pisa_abi.hip) is compiled with host sanitizers and
    linked to the regular kernel objects; tests/test_abi_sanitized.py runs the
    host-side ABI checks through it."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    obj = os.path.join(OBJ, "san", "pisa_abi.o")
    cmd = [HIPCC, *FLAGS, "-O1", "-g", *SAN_FLAGS, "-c", os.path.join(CSRC, "pisa_abi.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized ABI layer:\n{r.stderr}")
    kernels = [o for o in objs if not o.endswith("pisa_abi.hip.o")]
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", *kernels, obj, "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for the sanitized library:\n{r.stderr}")
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


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
    with cf.ThreadPoolExecutor(max_workers=len(UNITS)) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_c_caller(verbose)
    build_host_sanitized(objs, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
