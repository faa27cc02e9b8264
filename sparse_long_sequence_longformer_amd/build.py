"""Build liblfattn.so in-tree with hipcc for gfx950.

Usage: python -m sparse_long_sequence_longformer_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblfattn.so")

SOURCES = ["lf_attn.cpp", "lf_attn_kernels.hip", "lf_attn_bwd.hip", "lf_layer.hip"]
# Kernel arguments preloaded into scalar registers at wave launch (the leading scalar
# arguments of each kernel of the file, up to this many; a kernel whose first argument
# is a parameter struct gets none).  Firmware without preloading runs the compiler's
# own fallback, which loads them.
PRELOAD_ARGS = {"lf_attn_kernels.hip": 7, "lf_attn_bwd.hip": 9}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblfattn.so)")


ROCM_LIB = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-result",
        "-Wno-inline-asm",
        "-Wno-unused-const-variable",
        "-ffp-contract=fast",
        # keep MFMA accumulators in ordinary VGPRs (no AGPR copies around the softmax)
        "-mllvm", "-amdgpu-mfma-vgpr-form=true",
        # no packed fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    tmp = LIB + ".tmp"

    def compile_one(src):
        path = os.path.join(CSRC, src)
        obj = os.path.join(CSRC, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        pre = ["-mllvm", f"-amdgpu-kernarg-preload-count={PRELOAD_ARGS[src]}"] if src in PRELOAD_ARGS else []
        _run([cc, *compile_flags(), *pre, *lang, "-c", path, "-o", obj], verbose)
        return obj

    # the sources compile independently: one hipcc process each, at once
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    # hipBLASLt serves the layer's plain GEMMs
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, f"-L{ROCM_LIB}", "-lhipblaslt",
          f"-Wl,-rpath,{ROCM_LIB}"], verbose)
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    build_abi_check(verbose)
    return LIB


ABI_CHECK = os.path.join(PKG, "lf_abi_check")


def build_abi_check(verbose: bool = False) -> str:
    """A plain C program that calls the library through include/lf_attn.h only (built
    with the host C compiler against the HIP runtime; finds liblfattn.so beside it)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no C compiler for the C-ABI check program")
    rocm_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    tmp = ABI_CHECK + ".tmp"
    _run([cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", f"-I{rocm_inc}", f"-I{INCLUDE}",
          os.path.join(CSRC, "lf_abi_check.c"), "-o", tmp, f"-L{PKG}", "-llfattn", f"-L{ROCM_LIB}", "-lamdhip64",
          "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{ROCM_LIB}"], verbose)
    os.replace(tmp, ABI_CHECK)
    return ABI_CHECK


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
