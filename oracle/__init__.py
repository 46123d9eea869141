"""CPU oracle for C = ReLU(A.B) with fp16 inputs, fp32 accumulation and fp16 output.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package. The product
library never loads it; it shares no code with the GPU path.

What it computes is the quick-start kernel ``matmul_relu`` from the
"Programming model" section of the TileLang article (aiwiki.ai/wiki/tilelang):
an fp32 accumulator cleared, then A.B added over all of K, then ReLU on the
fp32 accumulator, then the copy-out to fp16. The arithmetic lives in
``oracle.c`` (plain C, no GPU code); this module builds it with gcc and calls
it through ctypes. Arrays are passed as numpy ``float16`` (or their ``uint16``
bit patterns) and are never converted by numpy on the way in or out.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off and no -ffast-math: the k accumulation must stay sequential.
CFLAGS = ["-O3", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-pthread", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it and return the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # TLG_ORACLE_LIB points the oracle at another build of oracle.c; the
        # planted-mistake tests use it to run the pins against mutated copies.
        path = os.environ.get("TLG_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_relu_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_relu_to_f16.restype = ctypes.c_uint16
        lib.oracle_f16_to_f32_array.argtypes = [p, p, i64]
        lib.oracle_f16_to_f32_array.restype = None
        lib.oracle_f32_to_f16_array.argtypes = [p, p, i64]
        lib.oracle_f32_to_f16_array.restype = None
        lib.oracle_gemm_relu_f16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, ctypes.c_int]
        lib.oracle_gemm_relu_f16.restype = ctypes.c_int
        lib.oracle_gemm_relu_f16_ijk.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
        lib.oracle_gemm_relu_f16_ijk.restype = None
        lib.oracle_gemm_relu_f16_elems.argtypes = [i64, p, i64, p, i64, i64, p, p, p]
        lib.oracle_gemm_relu_f16_elems.restype = None
        lib.oracle_default_threads.argtypes = []
        lib.oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _bits(x: np.ndarray) -> np.ndarray:
    """View an fp16 (or uint16) array as its uint16 bit patterns, no conversion."""
    if x.dtype == np.float16:
        return x.view(np.uint16)
    if x.dtype == np.uint16:
        return x
    raise TypeError(f"expected float16 or uint16 bit patterns, got {x.dtype}")


def _check_2d(x: np.ndarray, name: str) -> int:
    if x.ndim != 2:
        raise ValueError(f"{name} must be 2-D")
    if x.size == 0:
        return max(1, x.shape[1])  # nothing is read; an empty array's strides carry no layout
    if x.strides[1] != 2 or (x.shape[0] > 1 and x.strides[0] % 2):
        raise ValueError(f"{name} must be row-major with unit column stride")
    return x.strides[0] // 2 if x.shape[0] > 1 else max(1, x.shape[1])


def default_threads() -> int:
    """Threads the oracle uses by default: the CPUs in this process's affinity mask."""
    return int(_load().oracle_default_threads())


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact binary16 -> binary32 widening of every element (bit patterns in, float32 out)."""
    h = np.ascontiguousarray(_bits(np.asarray(h)))
    out = np.empty(h.shape, np.float32)
    _load().oracle_f16_to_f32_array(h.ctypes.data, out.ctypes.data, h.size)
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 round-to-nearest-even of every element; returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f32_to_f16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def relu_to_f16(acc: float) -> int:
    """The epilogue on one fp32 accumulator value: ReLU, then the fp16 copy-out."""
    return int(_load().oracle_relu_to_f16(float(acc)))


def gemm_relu(A: np.ndarray, B: np.ndarray, threads: int | None = None) -> np.ndarray:
    """C = ReLU(A.B) as fp16 (returned as uint16 bits), row-parallel, k ascending.

    A is (M, K) and B is (K, N), both fp16 (or uint16 bit patterns), row-major.
    Row views with a padded leading dimension are accepted.
    """
    A, B = _bits(A), _bits(B)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    lda, ldb = _check_2d(A, "A"), _check_2d(B, "B")
    C = np.zeros((M, N), np.uint16)
    rc = _load().oracle_gemm_relu_f16(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                      C.ctypes.data, max(1, N), int(threads or 0))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_relu_f16 failed with {rc}")
    return C


def gemm_relu_rows(A: np.ndarray, B: np.ndarray, rows, threads: int | None = None) -> np.ndarray:
    """Rows ``rows`` of ReLU(A.B): returns a (len(rows), N) uint16 array."""
    A = _bits(A)
    rows = np.asarray(rows, dtype=np.int64)
    sub = np.ascontiguousarray(A[rows, :])
    return gemm_relu(sub, B, threads)


def gemm_relu_ijk(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The literal i -> j -> k triple loop (single thread); uint16 bits out."""
    A, B = _bits(A), _bits(B)
    M, K = A.shape
    _, N = B.shape
    lda, ldb = _check_2d(A, "A"), _check_2d(B, "B")
    C = np.zeros((M, N), np.uint16)
    _load().oracle_gemm_relu_f16_ijk(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                     C.ctypes.data, max(1, N))
    return C


def gemm_relu_elems(A: np.ndarray, B: np.ndarray, ii, jj) -> np.ndarray:
    """C[ii[t], jj[t]] for each t, each from the literal definition; uint16 bits out."""
    A, B = _bits(A), _bits(B)
    K = A.shape[1]
    lda, ldb = _check_2d(A, "A"), _check_2d(B, "B")
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("ii and jj differ in shape")
    if ii.size and (ii.min() < 0 or ii.max() >= A.shape[0] or jj.min() < 0 or jj.max() >= B.shape[1]):
        raise IndexError("sample index out of range")
    out = np.empty(ii.shape, np.uint16)
    _load().oracle_gemm_relu_f16_elems(K, A.ctypes.data, lda, B.ctypes.data, ldb, ii.size,
                                       ii.ctypes.data, jj.ctypes.data, out.ctypes.data)
    return out


def gemm_relu_bt(A: np.ndarray, Bt: np.ndarray, threads: int | None = None) -> np.ndarray:
    """C = ReLU(A . Bt^T) for B given transposed (Bt is N x K): the same
    definition, with B read as Bt^T. The transpose is a copy of the bit
    patterns (no arithmetic); the sums are those of ``gemm_relu``."""
    Bt = np.asarray(Bt)
    return gemm_relu(A, np.ascontiguousarray(Bt.T), threads)


def gemm_relu_grouped(problems, trans_b: bool = False, threads: int | None = None) -> list:
    """Each problem (A, B) of a grouped call on its own: a list of C bit arrays."""
    f = gemm_relu_bt if trans_b else gemm_relu
    return [f(A, B, threads) for A, B in problems]
