"""Builds libfa.so (the C-ABI attention library) in-tree with hipcc for gfx950.

Usage: ``python -m causal_attention_fa_amd.build`` or ``build_library()``.
Every call compiles from source.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
# -amdgpu-mfma-vgpr-form=1: keep MFMA accumulators in architectural VGPRs;
#   the default heuristic parks the long-lived dK/dV accumulators in AGPRs and
#   then copies them to VGPRs and back around every tile's MFMAs.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I" + os.path.join(ROOT, "include"),
]


def source_fingerprint() -> str:
    """sha256 over the kernel sources, the public header and the compile flags: identifies
    the code a measurement (e.g. an HBM-traffic counter profile) was taken on."""
    import hashlib
    h = hashlib.sha256()
    h.update(" ".join(HIP_FLAGS[:-1]).encode())  # the include path differs between machines
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".cpp", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "fa.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libfa.so")
    return exe


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + HIP_FLAGS + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(extra_flags=(), verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_host_sanitized(out_dir: str, verbose: bool = False) -> str:
    """The C ABI's host code (fa_api.cpp) with stand-in launchers (fa_host_stubs.cpp:
    every launch reports an error), compiled by g++ with the address and
    undefined-behaviour sanitizers into ``out_dir/libfa_host_sanitized.so``.  It has no
    device code and computes nothing; it exists so that the argument checks can run
    under the sanitizers on a machine without a GPU.  Load it with the ASan runtime
    preloaded (``g++ -print-file-name=libasan.so``)."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libfa_host_sanitized.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_host_stubs.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host sanitizer build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build_library(sys.argv[1:], verbose=True)
