"""Pins for the oracle's layout and batching wrappers (no GPU).

``oracle.gemm_relu_bt`` (B given as its N x K transpose), ``oracle.
gemm_relu_grouped`` (a list of independent problems) and ``oracle.mx.
gemm_relu_mx_grouped`` add no arithmetic of their own: they hand each
problem, with B read the right way round, to the pinned fp16 and MX oracles.
What can go wrong in them is layout and bookkeeping: a dropped or doubled
transpose, problems returned in another order, a problem paired with another
problem's B or scales, the trans_b flag ignored. These pins compare each
wrapper, problem by problem, with references that share nothing with the
oracle: numpy's int64 matmul on integer-valued inputs (every partial sum is
an exact integer, so the result is rne16(relu(exact sum)) in any order), the
float64 error bound on uniform inputs, and numpy float64 on decoded MX
inputs. The ``check_*`` functions take the wrapper as an argument so that
the planted-mistake tests can run them against broken copies.

Grouped GEMM with a transposed B is listed among TileLang's milestones in the
zhichai.net forum post "TileLang: Writing Near-Hardware-Limit GPU Kernels in
70 Lines of Python" ("Key Technical Milestones"); the per-problem definition
is the quick-start kernel of the TileLang article (aiwiki.ai/wiki/tilelang,
"Programming model").
"""
import numpy as np
import pytest

import oracle
import oracle.mx as omx
from tiled_dense_gemm_06_amd import workloads as wl

from twin import relu_rne16_of_int

# Square (K == N) shapes are included on purpose: there a dropped transpose
# still yields a result of the right shape, which must then be wrong.
BT_SHAPES = [(7, 9, 9), (33, 40, 40), (64, 64, 64), (5, 17, 3), (31, 2, 130), (1, 1, 1), (9, 128, 72)]


def _int_inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    Bt = rng.integers(-2, 3, size=(N, K)).astype(np.float16)
    return A, Bt


def _exact_bt(A, Bt):
    return relu_rne16_of_int(A.astype(np.int64) @ Bt.astype(np.int64).T)


def check_bt(fn):
    """fn(A, Bt) must equal rne16(relu(A . Bt^T)) exactly on integer inputs,
    for ragged, square and padded-leading-dimension operands."""
    for M, N, K in BT_SHAPES:
        A, Bt = _int_inputs(M, N, K, seed=M * 131 + N * 7 + K)
        got = fn(A, Bt)
        assert got.shape == (M, N), (M, N, K)
        assert np.array_equal(got, _exact_bt(A, Bt)), (M, N, K)
    # row views of padded buffers (leading dimension above the row width)
    A, Bt = _int_inputs(19, 23, 37, seed=5)
    Ap = np.zeros((19, 48), np.float16)
    Bp = np.zeros((23, 45), np.float16)
    Ap[:, :37], Bp[:, :37] = A, Bt
    assert np.array_equal(fn(Ap[:, :37], Bp[:, :37]), _exact_bt(A, Bt))


def check_bt_float_bound(fn):
    """Uniform inputs: within the recursive-summation bound of the float64
    product A . Bt^T (numpy/BLAS), plus one fp16 ulp for the final rounding."""
    M, N, K = 40, 48, 48
    A, B = wl.make_random(M, N, K, seed=12, kind="uniform")
    Bt = np.ascontiguousarray(B.T)
    got = fn(A, Bt).view(np.float16).astype(np.float64)
    a, b = A.astype(np.float64), Bt.astype(np.float64)
    exact = a @ b.T
    gamma = K * 2.0**-24 / (1 - K * 2.0**-24)
    bound = gamma * (np.abs(a) @ np.abs(b).T) + 2.0**-10 * np.maximum(np.abs(exact), 2.0**-14)
    assert np.all(np.abs(got - np.maximum(exact, 0.0)) <= bound)


def _group_problems(trans_b, seed):
    """Problems of distinct shapes and, for two of them, one shared shape with
    different data (so a swap that keeps shapes still changes the results)."""
    shapes = [(5, 9, 11), (12, 12, 12), (12, 12, 12), (3, 30, 7), (17, 4, 64)]
    out = []
    for t, (M, N, K) in enumerate(shapes):
        A, Bt = _int_inputs(M, N, K, seed=seed + 17 * t)
        out.append((A, Bt if trans_b else np.ascontiguousarray(Bt.T)))
    return out


def check_grouped(fn):
    """fn(problems, trans_b) returns one result per problem, in order, each
    equal to that problem's exact result, with B read as given by trans_b."""
    for trans_b in (False, True):
        probs = _group_problems(trans_b, seed=3 if trans_b else 4)
        got = fn(probs, trans_b=trans_b)
        assert len(got) == len(probs)
        for t, ((A, B), C) in enumerate(zip(probs, got)):
            Bt = B if trans_b else np.ascontiguousarray(B.T)
            assert C.shape == (A.shape[0], Bt.shape[0]), (trans_b, t)
            assert np.array_equal(C, _exact_bt(A, Bt)), (trans_b, t)
    assert fn([], trans_b=False) == []


def _mx_ref(fmt, A, SA, Bt, SB):
    """numpy float64 over decoded, scaled elements (torch's float8 decoders),
    ReLU, numpy's fp16 cast: the reference of the MX oracle's own pins."""
    from test_oracle_mx_pins import ref_gemm

    return ref_gemm(fmt, A, SA, Bt, SB)


def _mx_group(fmt, seed):
    shapes = [(6, 10, 64), (9, 9, 96), (9, 9, 96), (2, 21, 32)]
    out = []
    for t, (M, N, K) in enumerate(shapes):
        A, SA, Bt, SB = wl.make_mx_inputs(fmt, M, N, K, seed=seed + 5 * t, kind="small_int")
        rng = np.random.default_rng(seed + 5 * t + 1)
        # distinct scales per block, row and problem, in a band that keeps sums exact
        SA = rng.integers(124, 131, size=SA.shape).astype(np.uint8)
        SB = rng.integers(124, 131, size=SB.shape).astype(np.uint8)
        out.append((A, SA, Bt, SB))
    return out


def check_mx_grouped(fn, fmt):
    """fn(fmt, problems) returns each problem's MX result, in order, equal to
    the float64 reference on that problem's own codes and scales."""
    probs = _mx_group(fmt, seed={"e4m3": 1, "e5m2": 2, "e2m1": 3}[fmt])
    got = fn(fmt, probs)
    assert len(got) == len(probs)
    for t, (p, C) in enumerate(zip(probs, got)):
        assert np.array_equal(C, _mx_ref(fmt, *p)), (fmt, t)


# ---------------------------------------------------------------- the wrappers as built

def test_gemm_relu_bt_exact_on_integer_inputs():
    check_bt(oracle.gemm_relu_bt)


def test_gemm_relu_bt_float_bound():
    check_bt_float_bound(oracle.gemm_relu_bt)


def test_gemm_relu_grouped_problem_by_problem():
    check_grouped(oracle.gemm_relu_grouped)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
def test_gemm_relu_mx_grouped_problem_by_problem(fmt):
    pytest.importorskip("torch")
    check_mx_grouped(omx.gemm_relu_mx_grouped, fmt)
