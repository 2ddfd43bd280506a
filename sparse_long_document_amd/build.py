"""Build the in-tree HIP library ``liblf_attn.so`` for gfx950.

Run ``python -m sparse_long_document_amd.build`` (or ``__graft_entry__.build()``).
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblf_attn.so")

SOURCES = ["lf_attn_host.cpp", "lf_attn_kernels.hip", "lf_attn_kernels_f16.hip", "lf_attn_kernels_d32.hip",
           "lf_attn_kernels_f16_d32.hip", "lf_attn_kernels_d128.hip", "lf_attn_kernels_f16_d128.hip", "lf_attn_bwd.hip",
           "lf_attn_bwd_f16.hip", "lf_proj.hip", "lf_attn_noalloc.hip"]

# Device code is built without packed fp32 instructions; the host pass of
# hipcc does not know the feature and warns, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, arch: str = "gfx950") -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out_path: str, verbose: bool = False) -> str:
    """The host part of the library alone (argument validation, workspace
    layout, launch planning: lf_attn_host.cpp) built with g++ under the
    address and undefined-behaviour sanitizers, the device entry points
    replaced by stubs that report no device (lf_host_stubs.cpp).  A CPU test
    runs the C-ABI tests against it (LF_ATTN_LIBRARY points the binding at
    it, and libasan is preloaded into that Python process)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", CSRC, "-I", os.path.join(rocm, "include"),
           os.path.join(CSRC, "lf_attn_host.cpp"), os.path.join(CSRC, "lf_host_stubs.cpp"),
           "-L", os.path.join(rocm, "lib"), "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64",
           "-o", out_path]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("g++ failed:\n" + r.stdout + r.stderr)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
