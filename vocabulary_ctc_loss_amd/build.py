"""Build libpcx.so (the HIP library behind include/pcx.h) for gfx950 in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpcx.so")
SOURCES = ["pcx_api.hip", "pcx_select.hip", "pcx_gemm.hip", "pcx_ctc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 math stays off on this target
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Werror", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed building libpcx.so")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


C_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi", "pcx_c_run.c")
C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi", "pcx_c_run")


def build_c_example(verbose: bool = False) -> str:
    """Compile the plain-C program that drives the C ABI in the tests (gcc,
    C11; HIP runtime API for device memory; libpcx.so found next to it by a
    relative runpath)."""
    rocm = os.path.dirname(os.path.dirname(HIPCC))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_EXAMPLE_SRC, "-L", HERE, "-lpcx", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../vocabulary_ctc_loss_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", C_EXAMPLE]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr + "\n")
        raise RuntimeError("gcc failed building the C ABI test program")
    return C_EXAMPLE


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_example(verbose=True))
