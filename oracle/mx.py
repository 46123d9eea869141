"""CPU oracle for the block-scaled (MX) variant of C = ReLU(A . B).

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module. It shares no code
with the GPU path or with the float16 oracle.

The arithmetic is in ``oracle_mx.c`` (its header states the definition and
the readings behind it: the hysenlabs.com project page on TileLang, "Three
backends under one language dialect", names FP4 E2M1 matrix cores on gfx950
and block-scaled MMA; the zhichai.net forum post on TileLang, "Key
Technical Milestones", names MXFP8 grouped GEMM with block scaling and a
transposed B; neither defines the scale semantics, which are read as the
OCP Microscaling formats: 32 elements along K share one E8M0 scale).

Arrays: A is (M, K) codes and B is (N, K) codes (B given transposed), as
uint8; for E2M1 two codes per byte (element 2t low nibble, 2t+1 high
nibble), so the arrays are (M, K/2) and (N, K/2) bytes. Scales are uint8
(M, K/32) and (N, K/32). Results are float16 bit patterns (uint16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import CFLAGS

E4M3, E5M2, E2M1 = 1, 2, 3
FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1}
BLOCK = 32

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_mx.c")
_LIB = os.path.join(_HERE, "liboracle_mx.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle_mx.c`` into ``liboracle_mx.so`` next to it and return the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # TLG_ORACLE_MX_LIB points at another build of oracle_mx.c (the
        # planted-mistake tests run the pins against mutated copies)
        path = os.environ.get("TLG_ORACLE_MX_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_mx_decode.argtypes = [i32, ctypes.c_uint32]
        lib.oracle_mx_decode.restype = ctypes.c_double
        lib.oracle_mx_scale.argtypes = [ctypes.c_uint32]
        lib.oracle_mx_scale.restype = ctypes.c_double
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_mx_relu_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_mx_relu_to_f16.restype = ctypes.c_uint16
        lib.oracle_gemm_relu_mx.argtypes = [i32, i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p, i64, i32]
        lib.oracle_gemm_relu_mx.restype = i32
        lib.oracle_gemm_relu_mx_elems.argtypes = [i32, i64, p, i64, p, i64, p, i64, p, i64, i64, p, p, p]
        lib.oracle_gemm_relu_mx_elems.restype = i32
        _lib = lib
    return _lib


def _fmt(fmt) -> int:
    f = FORMATS.get(fmt, fmt) if isinstance(fmt, str) else int(fmt)
    if f not in (E4M3, E5M2, E2M1):
        raise ValueError(f"unknown element format {fmt!r}")
    return f


def decode(fmt, code: int) -> float:
    """The value of one element code (binary64)."""
    return float(_load().oracle_mx_decode(_fmt(fmt), int(code)))


def scale_value(e: int) -> float:
    """The value of one E8M0 scale byte: 2^(e-127); 255 is NaN."""
    return float(_load().oracle_mx_scale(int(e)))


def f64_to_f16(x: float) -> int:
    """binary64 -> binary16 bits, round to nearest even."""
    return int(_load().oracle_f64_to_f16(float(x)))


def relu_to_f16(x: float) -> int:
    return int(_load().oracle_mx_relu_to_f16(float(x)))


def _rows(x: np.ndarray, name: str, elems_per_byte: int) -> int:
    """Leading dimension in elements of a C-contiguous 2-D uint8 array."""
    if x.dtype != np.uint8 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint8 array")
    if x.size and x.strides[1] != 1:
        raise ValueError(f"{name} must be row-major with unit column stride")
    ld_bytes = x.strides[0] if x.shape[0] > 1 and x.size else max(1, x.shape[1])
    return ld_bytes * elems_per_byte


def gemm_relu_mx(fmt, A: np.ndarray, SA: np.ndarray, Bt: np.ndarray, SB: np.ndarray,
                 threads: int | None = None) -> np.ndarray:
    """C = ReLU(sum over blocks of scale_a * scale_b * block dot product) as
    float16 bits, for A (M, K) and Bt (N, K) codes (packed for E2M1)."""
    f = _fmt(fmt)
    per = 2 if f == E2M1 else 1
    M, N = A.shape[0], Bt.shape[0]
    K = A.shape[1] * per
    if Bt.shape[1] * per != K:
        raise ValueError("inner dimensions differ")
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    if SA.shape != (M, K // BLOCK) or SB.shape != (N, K // BLOCK):
        raise ValueError("scale arrays must be (M, K/32) and (N, K/32)")
    lda, ldb = _rows(A, "A", per), _rows(Bt, "B", per)
    ldsa, ldsb = _rows(SA, "SA", 1), _rows(SB, "SB", 1)
    C = np.zeros((M, N), np.uint16)
    rc = _load().oracle_gemm_relu_mx(f, M, N, K, A.ctypes.data, lda, SA.ctypes.data, ldsa, Bt.ctypes.data, ldb,
                                     SB.ctypes.data, ldsb, C.ctypes.data, max(1, N), int(threads or 0))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_relu_mx failed with {rc}")
    return C


def gemm_relu_mx_elems(fmt, A, SA, Bt, SB, ii, jj) -> np.ndarray:
    """C[ii[t], jj[t]] for each t, each from the definition; float16 bits."""
    f = _fmt(fmt)
    per = 2 if f == E2M1 else 1
    K = A.shape[1] * per
    lda, ldb = _rows(A, "A", per), _rows(Bt, "B", per)
    ldsa, ldsb = _rows(SA, "SA", 1), _rows(SB, "SB", 1)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("ii and jj differ in shape")
    if ii.size and (ii.min() < 0 or ii.max() >= A.shape[0] or jj.min() < 0 or jj.max() >= Bt.shape[0]):
        raise IndexError("sample index out of range")
    out = np.empty(ii.shape, np.uint16)
    rc = _load().oracle_gemm_relu_mx_elems(f, K, A.ctypes.data, lda, SA.ctypes.data, ldsa, Bt.ctypes.data, ldb,
                                           SB.ctypes.data, ldsb, ii.size, ii.ctypes.data, jj.ctypes.data,
                                           out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_relu_mx_elems failed with {rc}")
    return out


def gemm_relu_mx_rows(fmt, A, SA, Bt, SB, rows, threads=None) -> np.ndarray:
    """Rows ``rows`` of the result: a (len(rows), N) uint16 array."""
    rows = np.asarray(rows, dtype=np.int64)
    return gemm_relu_mx(fmt, np.ascontiguousarray(A[rows]), np.ascontiguousarray(SA[rows]), Bt, SB, threads)


def gemm_relu_mx_grouped(fmt, problems, threads=None) -> list:
    """Each (A, SA, Bt, SB) problem of a grouped call on its own."""
    return [gemm_relu_mx(fmt, A, SA, Bt, SB, threads) for A, SA, Bt, SB in problems]
