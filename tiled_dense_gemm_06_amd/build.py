"""Builds libtlg.so (the C-ABI library and its gfx950 kernels) in place with hipcc.

Each source is compiled to its own object (in parallel), then the objects are
linked into the shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtlg.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "gemm_relu_gfx950.hip", "gemm_relu_pipe_gfx950.hip",
                                                 "gemm_relu_pipe16_gfx950.hip",
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
# Per-source flags. The 16 x 16 x 32 kernel's K step is one fully unrolled
# loop of 128 MFMA slots, larger than the unroller's default budget for a
# loop it is asked to unroll completely.
SOURCE_FLAGS = {
    "gemm_relu_pipe16_gfx950.hip": ["-mllvm", "-pragma-unroll-threshold=1000000"],
}


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def compile_cmd(output: str, extra=()) -> list[str]:
    """One hipcc command that builds the whole library from the sources
    (per-source flags are applied to every source)."""
    per = [f for flags in SOURCE_FLAGS.values() for f in flags]
    return [hipcc(), *HIP_FLAGS, *per, *extra, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", output]


def _compile_one(src: str, obj: str) -> subprocess.CompletedProcess:
    flags = [f for f in HIP_FLAGS if f != "-shared"]
    cmd = [hipcc(), *flags, *SOURCE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC,
           "-c", src, "-o", obj]
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    """Compile the library; always recompiles. Returns the path of libtlg.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in SOURCES]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile_one, SOURCES, objs))
    for src, r in zip(SOURCES, results):
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({r.returncode}):\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr:
            print(r.stderr)
    tmp = LIB + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
