"""Build libdg.so in-tree.

The host library (C++, HIP runtime + hipRTC) is compiled with the host C++
compiler against the ROCm headers, plus one HIP source (csrc/device.hip: the
library's status words and its measurement probes) compiled for gfx950 by
hipcc; the GEMM kernel source is embedded into the library as text and
compiled for gfx950 by hipRTC at run time, once per shape.  ``precompile()`` runs that hipRTC step ahead of time
(no GPU needed) so that the code objects of the standard workloads sit in the
in-tree cache and the device source is known to compile for gfx950.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
KERNEL = os.path.join(CSRC, "kernels", "fp8_gemm.hip")
INC = os.path.join(CSRC, "kernel_source.inc")
LIB = os.path.join(PKG, "libdg.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HOST_SOURCES = ["api.cpp", "jit.cpp", "heuristics.cpp"]
DEVICE_SOURCES = ["device.hip"]
BUILD_DIR = os.path.join(PKG, "_build")
# every HIP source is compiled for gfx950 with packed FP32 instructions off
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
DELIM = "DGSRC"


def write_kernel_include() -> None:
    src = open(KERNEL).read()
    if f'){DELIM}"' in src:
        raise RuntimeError("kernel source contains the raw-string delimiter")
    text = ("// generated from kernels/fp8_gemm.hip by build.py; do not edit\n"
            f'static const char kKernelSource[] = R"{DELIM}(' + src + f'){DELIM}";\n')
    old = open(INC).read() if os.path.exists(INC) else None
    if old != text:
        with open(INC, "w") as f:
            f.write(text)


def build_library(verbose: bool = False) -> str:
    write_kernel_include()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [os.path.join(ROCM, "bin", "hipcc"), *HIP_FLAGS, "-c",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cxx = os.environ.get("CXX", "g++")
    cmd = [cxx, "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in HOST_SOURCES], *objs,
           "-L", os.path.join(ROCM, "lib"), "-lhiprtc", "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


# kind, rows, N, K, groups, has_c: the five benchmark workloads (plus C variant) and the K-grouped one
STANDARD_SHAPES = [
    (0, 64, 2112, 7168, 1, 0),
    (0, 128, 24576, 1536, 1, 0),
    (0, 128, 24576, 1536, 1, 1),
    (0, 4096, 7168, 16384, 1, 0),
    (1, 32768, 4096, 7168, 4, 0),
    (2, 256, 7168, 2048, 4, 0),
    (3, 4096, 7168, 32768, 4, 0),     # K-grouped: the weight gradient of the contiguous workload
]


def precompile(shapes=STANDARD_SHAPES, num_cus: int = 256) -> None:
    """hipRTC-compile the kernels these shapes select into the cache (CPU only).

    torch is imported first so that the hipRTC library torch loads (the one a
    torch process resolves libdg.so's hipRTC dependency to) does the compiling
    and the cached code objects match what tests and the bench look up.
    """
    import ctypes
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB)
    lib.dg_precompile.restype = ctypes.c_int
    lib.dg_precompile.argtypes = [ctypes.c_int] * 7
    lib.dg_last_error.restype = ctypes.c_char_p
    for kind, rows, n, k, g, c in shapes:
        rc = lib.dg_precompile(kind, rows, n, k, g, c, num_cus)
        if rc != 0:
            raise RuntimeError(f"precompile {kind, rows, n, k, g, c} failed ({rc}): "
                               f"{lib.dg_last_error().decode()}")


if __name__ == "__main__":
    build_library(verbose=True)
    if "--precompile" in sys.argv:
        precompile()
