"""Builds libtlg.so (the C-ABI library and its gfx950 kernels) in place with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtlg.so")
SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "gemm_relu_gfx950.hip", "gemm_relu_pipe_gfx950.hip",
                                                 "gemm_relu_streamk_gfx950.hip", "gemm_relu_skinny_gfx950.hip",
                                                 "gemm_relu_mx_gfx950.hip", "gemm_relu_pingpong_gfx950.hip",
                                                 "noalloc.hip")]

# gfx950 only. Packed fp32 instructions are disabled for every GPU code path
# (the host pass reports the feature as unknown, which is harmless).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-inline-asm", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def compile_cmd(output: str, extra=()) -> list[str]:
    return [hipcc(), *HIP_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", output]


def build(verbose: bool = False) -> str:
    """Compile the library; always recompiles. Returns the path of libtlg.so."""
    tmp = LIB + ".tmp"
    r = subprocess.run(compile_cmd(tmp), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
