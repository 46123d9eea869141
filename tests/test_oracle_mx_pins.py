"""Pins for the block-scaled (MX) oracle (no GPU). Each test checks the oracle
against something other than itself: torch's own float8 and E8M0 decoders
(library routines), numpy's binary64 -> binary16 cast and float64 matmul,
hand-worked cases under tests/golden/, and invariants of the definition.

The definition pinned (stated in full in oracle/oracle_mx.c): blocks of 32
elements along K share one E8M0 scale 2^(e-127); C = ReLU(sum over blocks of
scale_a * scale_b * block dot product), rounded once to fp16. It is the
reading of the block-scaled GEMM named by the hysenlabs.com project page on
TileLang ("Three backends under one language dialect": FP4 E2M1 matrix
cores on gfx950, block-scaled MMA) and listed by the zhichai.net forum post
on TileLang ("Key Technical Milestones": MXFP8 grouped GEMM with block
scaling and a transposed B).
"""
import numpy as np
import pytest

import oracle.mx as mx
from conftest import read_golden
from tiled_dense_gemm_06_amd import workloads as wl

torch = pytest.importorskip("torch")

FMTS = ["e4m3", "e5m2", "e2m1"]


# ---------------------------------------------------------------- independent decoders

def _torch_decode8(fmt, codes):
    dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(dt).double().numpy()


def _e2m1_as_e4m3(codes):
    """E2M1 codes re-encoded as E4M3 bit patterns (same value): sign moves to
    bit 7; a normal exponent field e (bias 1) becomes e + 6 (bias 7) with the
    fraction bit moved to the top of the 3-bit fraction; the subnormal 0.5
    (field 0, fraction 1) is 2^-1, i.e. E4M3 field 6; zero stays zero."""
    codes = np.asarray(codes, dtype=np.int64)
    s, e, f = (codes >> 3) & 1, (codes >> 1) & 3, codes & 1
    body = np.where(e > 0, ((e + 6) << 3) | (f << 2), np.where(f == 1, 6 << 3, 0))
    return ((s << 7) | body).astype(np.uint8)


def ref_decode(fmt, codes):
    if fmt == "e2m1":
        return _torch_decode8("e4m3", _e2m1_as_e4m3(codes))
    return _torch_decode8(fmt, codes)


def unpack(fmt, X):
    """Codes per element (E2M1: element 2t is the low nibble of byte t)."""
    if fmt != "e2m1":
        return X.astype(np.int64)
    out = np.empty((X.shape[0], 2 * X.shape[1]), np.int64)
    out[:, 0::2] = X & 0xF
    out[:, 1::2] = X >> 4
    return out


def ref_gemm(fmt, A, SA, Bt, SB):
    """numpy float64 matmul over decoded, scaled elements, ReLU, numpy's fp16 cast."""
    a = ref_decode(fmt, unpack(fmt, A)) * np.repeat(np.exp2(SA.astype(np.float64) - 127), 32, axis=1)
    b = ref_decode(fmt, unpack(fmt, Bt)) * np.repeat(np.exp2(SB.astype(np.float64) - 127), 32, axis=1)
    c = a @ b.T
    with np.errstate(over="ignore"):  # sums beyond 65520 become inf, as in the definition
        return np.where(c > 0, c, 0.0).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- conversions

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_decode_8bit_exhaustive_vs_torch(fmt):
    codes = np.arange(256)
    ours = np.array([mx.decode(fmt, c) for c in codes])
    ref = _torch_decode8(fmt, codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))  # -0 stays -0


def test_e8m0_exhaustive_vs_torch():
    codes = np.arange(256)
    ours = np.array([mx.scale_value(c) for c in codes])
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_e2m1_values():
    ours = np.array([mx.decode("e2m1", c) for c in range(16)])
    assert np.array_equal(ours, ref_decode("e2m1", np.arange(16)))
    pos = ours[:8]
    assert np.all(np.diff(pos) > 0) and pos[0] == 0 and pos[-1] == 6.0  # ordered codes, largest 6
    assert np.array_equal(ours[8:], -pos) and np.signbit(ours[8])          # sign bit, -0
    assert np.all(2 * pos == np.round(2 * pos))                              # multiples of 1/2


def test_f64_to_f16_vs_numpy():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(50000) * np.exp2(rng.integers(-30, 18, 50000))
    # exact ties at every binade and at the subnormal quantum, and the edges
    m = rng.integers(1024, 2048, 2000)
    e = rng.integers(-24, 16, 2000)
    ties = (2 * m + 1) * np.exp2(e.astype(np.float64) - 11)
    edges = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-14,
                      2.0**-14 - 2.0**-25, 1e-300, -1e300, np.inf, -np.inf])
    for arr in (x, ties, edges):
        with np.errstate(over="ignore"):
            ref = arr.astype(np.float16).view(np.uint16)
        ours = np.array([mx.f64_to_f16(v) for v in arr], dtype=np.uint16)
        assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- the GEMM

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(7, 9, 64), (33, 17, 256), (1, 40, 512)])
def test_unit_scales_vs_numpy(fmt, shape):
    M, N, K = shape
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, M, N, K, seed=M * 7 + N + K, kind="random")
    SA[:] = 127
    SB[:] = 127
    assert np.array_equal(mx.gemm_relu_mx(fmt, A, SA, Bt, SB), ref_gemm(fmt, A, SA, Bt, SB))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(5, 11, 96), (31, 29, 320)])
def test_block_scales_vs_numpy(fmt, shape):
    M, N, K = shape
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, M, N, K, seed=M + N * 3 + K, kind="random", spread=4)
    assert np.array_equal(mx.gemm_relu_mx(fmt, A, SA, Bt, SB), ref_gemm(fmt, A, SA, Bt, SB))


def _golden_case(line):
    head, elems, sa, sb, want = [p.strip() for p in line.split("|")]
    fmt, K = head.split()
    K = int(K)
    a = np.zeros((1, K), np.int64)
    b = np.zeros((1, K), np.int64)
    for item in elems.split():
        k, ac, bc = item.split(":")
        a[0, int(k)], b[0, int(k)] = int(ac, 16), int(bc, 16)
    if fmt == "e2m1":
        a = a[:, 0::2] | (a[:, 1::2] << 4)
        b = b[:, 0::2] | (b[:, 1::2] << 4)
    SA = np.array([[int(v) for v in sa.split()]], np.uint8)
    SB = np.array([[int(v) for v in sb.split()]], np.uint8)
    return fmt, a.astype(np.uint8), SA, b.astype(np.uint8), SB, int(want, 16)


def test_worked_examples():
    lines = read_golden("mx_worked_examples.txt")
    assert len(lines) == 7
    for line in lines:
        fmt, A, SA, Bt, SB, want = _golden_case(line)
        got = int(mx.gemm_relu_mx(fmt, A, SA, Bt, SB)[0, 0])
        assert got == want, f"{line}: got {got:04x}"
        assert int(mx.gemm_relu_mx_elems(fmt, A, SA, Bt, SB, [0], [0])[0]) == want


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_shift_doubles_exactly(fmt):
    """Raising every scale of A's row i by one doubles that row of the
    unrounded sum; away from overflow and the subnormal range the fp16
    result doubles exactly (its bits gain 0x400)."""
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, 6, 10, 128, seed=9, kind="random")
    C0 = mx.gemm_relu_mx(fmt, A, SA, Bt, SB)
    SA2 = SA.copy()
    SA2[2] += 1
    C1 = mx.gemm_relu_mx(fmt, A, SA2, Bt, SB)
    assert np.array_equal(np.delete(C0, 2, 0), np.delete(C1, 2, 0))
    row0, row1 = C0[2].astype(np.int64), C1[2].astype(np.int64)
    normal = (row0 >= 0x0400) & (row0 < 0x7800)
    assert normal.sum() >= 3
    assert np.array_equal(row1[normal], row0[normal] + 0x400)
    assert np.all(row1[row0 == 0] == 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_integer_inputs_and_specials(fmt):
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, 9, 13, 256, seed=4, kind="small_int")
    ai = ref_decode(fmt, unpack(fmt, A)).astype(np.int64)
    bi = ref_decode(fmt, unpack(fmt, Bt)).astype(np.int64)
    exact = np.maximum(ai @ bi.T, 0)  # int64 matmul; |sums| <= 1024, exact in fp16 only when small
    got = mx.gemm_relu_mx(fmt, A, SA, Bt, SB)
    assert np.array_equal(got, exact.astype(np.float16).view(np.uint16))
    # a NaN scale (byte 255) makes the sum NaN, and ReLU maps NaN to +0
    SA2 = SA.copy()
    SA2[0, 3] = 255
    got2 = mx.gemm_relu_mx(fmt, A, SA2, Bt, SB)
    assert np.all(got2[0] == 0) and np.array_equal(got2[1:], got[1:])
    # K = 0: the empty sum, +0 everywhere
    z = np.zeros((4, 0), np.uint8)
    assert np.all(mx.gemm_relu_mx(fmt, z, np.zeros((4, 0), np.uint8), np.zeros((3, 0), np.uint8),
                                  np.zeros((3, 0), np.uint8)) == 0)


def test_rows_elems_and_threads_agree():
    A, SA, Bt, SB = wl.make_mx_inputs("e4m3", 40, 24, 192, seed=2)
    full = mx.gemm_relu_mx("e4m3", A, SA, Bt, SB)
    assert np.array_equal(full, mx.gemm_relu_mx("e4m3", A, SA, Bt, SB, threads=1))
    rows = [0, 7, 39]
    assert np.array_equal(mx.gemm_relu_mx_rows("e4m3", A, SA, Bt, SB, rows), full[rows])
    ii, jj = np.array([0, 5, 39, 12]), np.array([0, 23, 7, 12])
    assert np.array_equal(mx.gemm_relu_mx_elems("e4m3", A, SA, Bt, SB, ii, jj), full[ii, jj])


def test_rejects_bad_arguments():
    A, SA, Bt, SB = wl.make_mx_inputs("e4m3", 4, 4, 64, seed=1)
    with pytest.raises(ValueError):
        mx.gemm_relu_mx("e4m3", A[:, :48], SA, Bt, SB)  # K not a multiple of 32 / shapes differ
    with pytest.raises(ValueError):
        mx.gemm_relu_mx("e4m3", A, SA[:, :1], Bt, SB)
    with pytest.raises(ValueError):
        mx.gemm_relu_mx("fp7", A, SA, Bt, SB)
