"""Seeded synthetic workloads for the fp16 GEMM+ReLU path.

This module only draws inputs. It performs none of the method's arithmetic, so
both the GPU path and the CPU oracle can take their inputs from it.

Shapes follow the quick-start kernel of the TileLang article (aiwiki.ai/wiki/
tilelang, "Programming model": A is (M, K) fp16, B is (K, N) fp16, both
row-major). The five workloads are a tiny square case, a mid-size square
case, a ragged case whose sizes are multiples of no tile size, a skinny
memory-bound case (M = 16), and the 8192-cubed compute-bound case.

Recipe (fixed, so the inputs are reproducible anywhere):
  * ``numpy.random.default_rng(seed)`` (PCG64);
  * A is drawn first, then B, each in one call, row-major, as float64;
  * each is cast once to float16 (round to nearest even) with ``astype``;
  * uniform is ``rng.uniform(-1, 1)``; normal is ``rng.normal(0, std)`` with the
    second parameter read as the standard deviation; the integer variant draws
    ``rng.integers(-2, 3)`` (values -2..2) from the same seed.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Dist:
    kind: str          # "uniform" | "normal"
    scale: float = 1.0  # uniform: half-width; normal: standard deviation


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    a: Dist
    b: Dist
    description: str

    @property
    def flop(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def alg_bytes(self) -> int:
        """A, B and C fp16 footprints, each read or written once."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)


_U = Dist("uniform", 1.0)

WORKLOADS = {
    w.name: w
    for w in [
        Workload("square256", 256, 256, 256, 0, _U, _U,
                 "M=N=K=256, U[-1,1] from seed 0"),
        Workload("square4096", 4096, 4096, 4096, 1, _U, _U,
                 "M=N=K=4096, U[-1,1] from seed 1"),
        Workload("ragged3001x2049x1537", 3001, 2049, 1537, 2,
                 Dist("normal", 1.0 / math.sqrt(1537)), Dist("normal", 1.0 / math.sqrt(1537)),
                 "M=3001 N=2049 K=1537, N(0, std 1/sqrt(K)) from seed 2"),
        Workload("skinny16x14336x4096", 16, 14336, 4096, 3, _U, Dist("normal", 0.02),
                 "M=16 N=14336 K=4096, A U[-1,1], B N(0, std 0.02) from seed 3"),
        Workload("square8192", 8192, 8192, 8192, 4, _U, _U,
                 "M=N=K=8192, U[-1,1] from seed 4"),
        # not one of the pages' configurations: a decode batch between one and
        # two 32-row MFMA blocks, measured with bench.py --workload
        Workload("decode48x4096x14336", 48, 4096, 14336, 5, _U, Dist("normal", 0.02),
                 "M=48 N=4096 K=14336, A U[-1,1], B N(0, std 0.02) from seed 5"),
    ]
}

ORDER = ["square256", "square4096", "ragged3001x2049x1537", "skinny16x14336x4096", "square8192"]


def _draw(rng: np.random.Generator, shape, dist: Dist, integer: bool) -> np.ndarray:
    if integer:
        x = rng.integers(-2, 3, size=shape)
    elif dist.kind == "uniform":
        x = rng.uniform(-dist.scale, dist.scale, size=shape)
    elif dist.kind == "normal":
        x = rng.normal(0.0, dist.scale, size=shape)
    else:
        raise ValueError(dist.kind)
    return x.astype(np.float16)


def make_inputs(w: Workload | str, integer: bool = False, seed: int | None = None):
    """Return (A, B) as C-contiguous float16 arrays of shapes (M, K) and (K, N)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    A = _draw(rng, (w.M, w.K), w.a, integer)
    B = _draw(rng, (w.K, w.N), w.b, integer)
    return A, B


def make_random(M: int, N: int, K: int, seed: int, kind: str = "uniform"):
    """Inputs of any shape for sweeps: kind is 'uniform' (U[-1,1]), 'normal'
    (std 1/sqrt(K)), 'integer' (-2..2) or 'integer_pos' (0..3, whose sums
    reach the thousands and so exercise the fp16 rounding of the output)."""
    rng = np.random.default_rng(seed)
    if kind == "integer":
        return _draw(rng, (M, K), _U, True), _draw(rng, (K, N), _U, True)
    if kind == "integer_pos":
        return (rng.integers(0, 4, size=(M, K)).astype(np.float16),
                rng.integers(0, 4, size=(K, N)).astype(np.float16))
    if kind == "normal":
        d = Dist("normal", 1.0 / math.sqrt(max(K, 1)))
        return _draw(rng, (M, K), d, False), _draw(rng, (K, N), d, False)
    return _draw(rng, (M, K), _U, False), _draw(rng, (K, N), _U, False)


def sha256(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


# ---------------------------------------------------------------------------
# Block-scaled (MX) inputs: element codes and E8M0 scale bytes, drawn as bit
# fields (no decoding and no GEMM arithmetic here).
#
# Recipe: ``numpy.random.default_rng(seed)``; A's codes, then B's codes, then
# A's scales, then B's scales, each in the calls below, row-major. B is drawn
# as its transpose, N x K (the block-scaled path takes B that way).
#  * kind "random": per element a sign bit (uniform), an exponent field
#    (uniform over bias-3 .. bias+3 for the 8-bit formats, over 0..3 for
#    E2M1), and a fraction field (uniform); then one element in 16 gets
#    exponent field 0 (zero or subnormal). Scales uniform over
#    127-spread .. 127+spread (2^-spread .. 2^spread).
#  * kind "small_int": elements -2, -1, 0, 1, 2 (uniform), encoded as
#    sign | (bias + log2|v|) << fraction bits, 0 as code 0; all scales 127
#    (2^0), so every sum is an integer that fp32 holds exactly.
# E2M1 codes are packed two per byte: element 2t in the low nibble.
# ---------------------------------------------------------------------------

MX_FORMATS = {"e4m3": (4, 3), "e5m2": (5, 2), "e2m1": (2, 1)}  # exponent bits, fraction bits
MX_BLOCK = 32


def _mx_codes(rng: np.random.Generator, shape, fmt: str, kind: str) -> np.ndarray:
    eb, mb = MX_FORMATS[fmt]
    bias = (1 << (eb - 1)) - 1
    sign = rng.integers(0, 2, size=shape, dtype=np.int64) << (eb + mb)
    if kind == "small_int":
        mag = rng.integers(0, 3, size=shape, dtype=np.int64)  # |v| = 0, 1, 2
        expf = np.where(mag == 0, 0, bias + (mag == 2))
        codes = np.where(mag == 0, 0, sign | (expf << mb))
    elif kind == "random":
        lo, hi = (0, (1 << eb) - 1) if fmt == "e2m1" else (bias - 3, bias + 3)
        expf = rng.integers(lo, hi + 1, size=shape, dtype=np.int64)
        frac = rng.integers(0, 1 << mb, size=shape, dtype=np.int64)
        expf = np.where(rng.integers(0, 16, size=shape) == 0, 0, expf)
        codes = sign | (expf << mb) | frac
    else:
        raise ValueError(kind)
    codes = codes.astype(np.uint8)
    if fmt == "e2m1":
        codes = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(codes)


def make_mx_inputs(fmt: str, M: int, N: int, K: int, seed: int, kind: str = "random", spread: int = 2):
    """(A, SA, Bt, SB): A codes (M, K) and Bt codes (N, K) as uint8 (E2M1:
    (M, K/2) and (N, K/2) packed bytes), scales (M, K/32) and (N, K/32)."""
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    A = _mx_codes(rng, (M, K), fmt, kind)
    Bt = _mx_codes(rng, (N, K), fmt, kind)
    if kind == "small_int":
        SA = np.full((M, K // MX_BLOCK), 127, np.uint8)
        SB = np.full((N, K // MX_BLOCK), 127, np.uint8)
    else:
        SA = rng.integers(127 - spread, 128 + spread, size=(M, K // MX_BLOCK)).astype(np.uint8)
        SB = rng.integers(127 - spread, 128 + spread, size=(N, K // MX_BLOCK)).astype(np.uint8)
    return A, SA, Bt, SB
