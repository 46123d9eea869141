"""CPU emulation of the gfx950 kernels' data movement (tests/emu/tile_emu.cpp),
built on the kernels' own index arithmetic, checked against the oracle.

This runs without a GPU. It catches indexing mistakes (a wrong swizzle, a
lane fetching the wrong chunk, an out-of-bounds global access, an LDS byte
written twice, a C element written twice or never, a bank conflict in a
fragment read) before any kernel is launched on hardware.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tiled_dense_gemm_06_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "emu", "tile_emu.cpp")
CSRC = os.path.join(ROOT, "tiled_dense_gemm_06_amd", "csrc")

ERR_NAMES = ["oob_global", "lds_multi", "lds_oob", "bank_conflict", "c_multi", "c_missing", "c_outside", "tile_dup"]
# config ids understood by emu_gemm_relu (mirroring the kernels' tile tables; 3 is
# the 64-deep two-stage layout of the pipelined kernel, 6 and 7 its half tiles)
DMA_CONFIGS = {0: (256, 256, 32), 1: (128, 128, 32), 2: (64, 64, 64), 3: (256, 256, 64), 4: (256, 256, 64),
               5: (256, 256, 32), 6: (256, 128, 64), 7: (128, 256, 64)}
SPLIT_CONFIGS = {10: (32, 128, 64), 11: (32, 256, 64)}


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    out = tmp_path_factory.mktemp("emu") / "libtile_emu.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, SRC, "-o", str(out)], check=True)
    L = ctypes.CDLL(str(out))
    p, i, l = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
    L.emu_gemm_relu.argtypes = [i, i, i, i, p, l, p, l, p, l, i, i, p, p]
    L.emu_gemm_relu.restype = i
    L.emu_check_remap.argtypes = [i]
    L.emu_check_remap.restype = l
    L.emu_check_streamk.argtypes = [l, i, i]
    L.emu_check_streamk.restype = l
    L.emu_check_strip_sk.argtypes = [i, i, i]
    L.emu_check_strip_sk.restype = l
    L.emu_check_epilogue.argtypes = [i]
    L.emu_gemm_relu_bt.argtypes = [i, i, i, i, p, l, p, l, p, l, p]
    L.emu_gemm_relu_bt.restype = i
    L.emu_check_epilogue.restype = l
    return L


def run_emu(L, config, A, B, splits=1, k_split=0):
    M, K = A.shape
    N = B.shape[1]
    C = np.full((M, N), 0xFFFF, np.uint16)
    W = np.zeros(max(1, splits * M * N), np.float32)
    errs = np.zeros(8, np.int64)
    A16, B16 = np.ascontiguousarray(A.view(np.uint16)), np.ascontiguousarray(B.view(np.uint16))
    rc = L.emu_gemm_relu(config, M, N, K, A16.ctypes.data, K, B16.ctypes.data, N, C.ctypes.data, N,
                         splits, k_split, W.ctypes.data, errs.ctypes.data)
    assert rc == 0
    return C, dict(zip(ERR_NAMES, errs.tolist()))


def test_xcd_remap_is_bijection(emu):
    assert emu.emu_check_remap(2100) == 0


@pytest.mark.parametrize("tiles,ipt,G", [(112, 64, 512), (1, 1, 1), (1, 8, 8), (3, 5, 7), (7, 3, 21), (112, 64, 100),
                                         (4, 128, 512), (512, 2, 512), (37, 11, 96)])
def test_streamk_ranges(emu, tiles, ipt, G):
    total = tiles * ipt
    assert emu.emu_check_streamk(total, min(G, total), ipt) == 0


@pytest.mark.parametrize("strips,nkb,G", [(224, 64, 256), (224, 64, 512), (128, 128, 256), (5, 64, 256),
                                          (1, 1, 256), (1, 7, 1), (3, 1, 256), (100, 7, 256), (256, 64, 256),
                                          (17, 3, 40), (64, 16, 512), (255, 9, 256)])
def test_strip_streamk_segments(emu, strips, nkb, G):
    """The stream-K strip kernel's ranges, parts, counts and partial slots
    (its segment arithmetic from the shared index header)."""
    assert emu.emu_check_strip_sk(strips, nkb, G) == 0


@pytest.mark.parametrize("config", sorted(DMA_CONFIGS))
def test_lds_epilogue_index_math(emu, config):
    """The C epilogue through LDS (wave blocks of 128, 64 and 32 columns):
    every result register reaches its own C position, each LDS piece is
    written once, and neither the writes nor the read-back have bank
    conflicts."""
    assert emu.emu_check_epilogue(config) == 0


# shapes that satisfy the direct-to-LDS conditions (K % 8 == 0, N % 8 == 0), several tiles, ragged tails
SHAPES = [(64, 64, 64), (200, 136, 88), (257, 264, 520), (70, 512, 40), (1, 8, 8), (300, 40, 16)]


@pytest.mark.parametrize("config", [0, 1, 2, 3, 4, 20, 21, 23])
@pytest.mark.parametrize("shape", SHAPES + [(301, 259, 203), (65, 70, 9), (130, 129, 1), (300, 264, 200),
                                            (257, 9, 4104), (513, 520, 72)])
def test_transposed_b_tiles_match_oracle_integer(emu, config, shape):
    """B given transposed (N x K): its tile is loaded and read like A's; the
    ragged K tail is staged the same way. Any K and N work (configurations
    20, 21, 23: the 16 x 16 x 32 pipelined tiles, 256 x 256, 128 x 256 and
    192 x 256)."""
    M, N, K = shape
    A, B = wl.make_random(M, N, K, seed=M + 3 * N + K, kind="integer_pos" if K > 100 else "integer")
    Bt = np.ascontiguousarray(B.T)
    C = np.full((M, N), 0xFFFF, np.uint16)
    errs = np.zeros(8, np.int64)
    A16, Bt16 = np.ascontiguousarray(A.view(np.uint16)), Bt.view(np.uint16)
    rc = emu.emu_gemm_relu_bt(config, M, N, K, A16.ctypes.data, K, Bt16.ctypes.data, K, C.ctypes.data, N,
                              errs.ctypes.data)
    assert rc == 0
    errs = dict(zip(ERR_NAMES, errs.tolist()))
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C, oracle.gemm_relu(A, B))


@pytest.mark.parametrize("config", sorted(DMA_CONFIGS))
@pytest.mark.parametrize("shape", SHAPES)
def test_dma_tiles_match_oracle_integer(emu, config, shape):
    M, N, K = shape
    A, B = wl.make_random(M, N, K, seed=M + N + K, kind="integer_pos" if K > 100 else "integer")
    C, errs = run_emu(emu, config, A, B)
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C, oracle.gemm_relu(A, B))


@pytest.mark.parametrize("shape", [(48, 64, 128), (64, 136, 520), (33, 392, 64), (1, 8, 8), (63, 200, 1000)])
def test_one_wave_strip_tile_matches_oracle_integer(emu, shape):
    """The 64-row strip's ring layout (one wave loads and multiplies a whole
    64 x 64 x 64 block: eight 1 KiB loads of A and of B, 2 x 2 MFMA tiles),
    emulated over the problem's strips: loads in bounds, each LDS byte written
    once, no bank conflicts, exact result."""
    M, N, K = shape
    A, B = wl.make_random(M, N, K, seed=M + 2 * N + K, kind="integer_pos" if K > 100 else "integer")
    C, errs = run_emu(emu, 8, A, B)
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C, oracle.gemm_relu(A, B))


@pytest.mark.parametrize("shape", [(48, 64, 128), (64, 136, 520), (33, 392, 64), (1, 8, 8), (63, 200, 1000)])
def test_one_wave_strip_tile_transposed_b(emu, shape):
    """The same strip ring with B given transposed (N x K): each block of B is
    64 rows n of 64 k, loaded with A's chunk order and swizzle and read with
    A's fragment reads; loads in bounds, each LDS byte written once, no bank
    conflicts, exact result."""
    M, N, K = shape
    A, B = wl.make_random(M, N, K, seed=M + 3 * N + K, kind="integer_pos" if K > 100 else "integer")
    Bt = np.ascontiguousarray(B.T)
    C = np.full((M, N), 0xFFFF, np.uint16)
    errs = np.zeros(8, np.int64)
    A16, Bt16 = np.ascontiguousarray(A.view(np.uint16)), Bt.view(np.uint16)
    rc = emu.emu_gemm_relu_bt(8, M, N, K, A16.ctypes.data, K, Bt16.ctypes.data, K, C.ctypes.data, N,
                              errs.ctypes.data)
    assert rc == 0
    errs = dict(zip(ERR_NAMES, errs.tolist()))
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C, oracle.gemm_relu(A, B))


RAGGED = [(301, 259, 203), (65, 9, 17), (130, 264, 97), (33, 41, 8), (257, 131, 1), (64, 64, 65), (3, 263, 72)]


@pytest.mark.parametrize("config", sorted(DMA_CONFIGS))
@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_tiles_match_oracle_integer(emu, config, shape):
    """K or N not a multiple of 8, odd leading dimensions: the loads stop at
    the largest multiple of 8 below K, a chunk crossing the N edge reads into
    the next row of B (never past the last row), and the last rows come from
    a staged zero-padded block."""
    M, N, K = shape
    A, B = wl.make_random(M, N, K, seed=M * 7 + N * 3 + K, kind="integer_pos")
    C, errs = run_emu(emu, config, A, B)
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C, oracle.gemm_relu(A, B))


@pytest.mark.parametrize("config", sorted(DMA_CONFIGS))
def test_dma_tiles_uniform_within_tolerance(emu, config):
    A, B = wl.make_random(130, 264, 96, seed=5)
    C, errs = run_emu(emu, config, A, B)
    assert all(v == 0 for v in errs.values()), errs
    ref = oracle.gemm_relu(A, B).view(np.float16).astype(np.float64)
    got = C.view(np.float16).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-2 + 4e-3 * np.abs(ref))


@pytest.mark.parametrize("config", sorted(SPLIT_CONFIGS))
@pytest.mark.parametrize("shape,splits", [((16, 512, 1024), 4), ((5, 264, 512), 3), ((40, 128, 192), 2)])
def test_splitk_matches_oracle_integer(emu, config, shape, splits):
    M, N, K = shape
    bk = SPLIT_CONFIGS[config][2]
    ksteps = -(-K // bk)
    k_split = -(-ksteps // splits) * bk
    splits = -(-K // k_split)
    A, B = wl.make_random(M, N, K, seed=7, kind="integer_pos")
    C, errs = run_emu(emu, config, A, B, splits=splits, k_split=k_split)
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C, oracle.gemm_relu(A, B))


# ---------------------------------------------------------------- block-scaled (MX) kernel

import oracle.mx as omx  # noqa: E402

_HW = {"e4m3": 0, "e5m2": 1, "e2m1": 4}


def run_emu_mx(L, config, fmt, A, SA, Bt, SB):
    M, N = A.shape[0], Bt.shape[0]
    K = A.shape[1] * (2 if fmt == "e2m1" else 1)
    C = np.full((M, N), 0x7E00, np.uint16)
    errs = np.zeros(8, np.int64)
    p = ctypes.c_void_p
    L.emu_gemm_relu_mx.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, p,
                                   ctypes.c_long, p, ctypes.c_long, p, ctypes.c_long, p, ctypes.c_long, p,
                                   ctypes.c_long, p]
    rc = L.emu_gemm_relu_mx(config, _HW[fmt], M, N, K, A.ctypes.data, A.shape[1], SA.ctypes.data, SA.shape[1],
                            Bt.ctypes.data, Bt.shape[1], SB.ctypes.data, SB.shape[1], C.ctypes.data, N,
                            errs.ctypes.data)
    assert rc == 0
    return C, errs


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
@pytest.mark.parametrize("config,shape", [(1, (130, 136, 256)), (1, (1, 8, 128)), (1, (300, 200, 384)),
                                          (0, (257, 260, 256)), (0, (256, 256, 128))])
def test_mx_tiles_match_oracle_integer(emu, fmt, config, shape):
    """The block-scaled kernel's loads, scale dwords, fragment and scale reads
    and MFMA lane semantics, emulated on the CPU: every access in bounds, no
    LDS bank conflict, every C element written once, and with integer codes
    and block scales 2^-4..2^4 (exact sums) the oracle's bits exactly."""
    M, N, K = shape
    A, _, Bt, _ = wl.make_mx_inputs(fmt, M, N, K, seed=M + N + K, kind="small_int")
    rng = np.random.default_rng(M * N + K)
    SA = rng.integers(123, 132, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(123, 132, size=(N, K // 32)).astype(np.uint8)
    C, errs = run_emu_mx(emu, config, fmt, A, SA, Bt, SB)
    assert not errs.any(), errs
    assert np.array_equal(C, omx.gemm_relu_mx(fmt, A, SA, Bt, SB))


# the 16 x 16 x 32 pipelined kernel: four waves of 128 x 128 (20), the 128 x 256
# half tiles (21), eight waves of 128 x 64 (22), 192 x 256 tiles (23)
PIPE16_CONFIGS = [20, 21, 22, 23]
PIPE16_SHAPES = [(256, 256, 64), (300, 264, 192), (200, 264, 200), (130, 300, 203), (64, 256, 40), (257, 9, 520),
                 (1, 8, 8), (513, 40, 136)]


def run_emu_ld(L, config, A, B, lda, ldb, ldc):
    """Like run_emu, with A, B and C held in padded rows."""
    M, K = A.shape
    N = B.shape[1]
    Ap = np.full((M, lda), 0x7E00, np.uint16)  # NaN padding: a read of it would show in C
    Ap[:, :K] = A.view(np.uint16)
    Bp = np.full((K, ldb), 0x7E00, np.uint16)
    Bp[:, :N] = B.view(np.uint16)
    C = np.full((M, ldc), 0xFFFF, np.uint16)
    W = np.zeros(1, np.float32)
    errs = np.zeros(8, np.int64)
    rc = L.emu_gemm_relu(config, M, N, K, Ap.ctypes.data, lda, Bp.ctypes.data, ldb, C.ctypes.data, ldc,
                         1, 0, W.ctypes.data, errs.ctypes.data)
    assert rc == 0
    return C, dict(zip(ERR_NAMES, errs.tolist()))


@pytest.mark.parametrize("config", PIPE16_CONFIGS)
@pytest.mark.parametrize("shape", PIPE16_SHAPES)
def test_pipe16_tiles_match_oracle_integer(emu, config, shape):
    """The 16 x 16 x 32 kernel's own load offsets, buffer ranges, fragment
    addresses, K tail and epilogue: every global read inside its matrix, each
    LDS byte written once per stage, conflict-free fragment and epilogue
    accesses, every C element written once, and C bit-exact with the oracle
    on integer inputs."""
    M, N, K = shape
    A, B = wl.make_random(M, N, K, seed=M * 7 + N * 3 + K, kind="integer")
    C, errs = run_emu(emu, config, A, B)
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C, oracle.gemm_relu(A, B))


@pytest.mark.parametrize("config", PIPE16_CONFIGS)
@pytest.mark.parametrize("shape,lds", [((300, 264, 192), (200, 272, 280)), ((130, 300, 203), (211, 305, 301)),
                                       ((257, 9, 520), (520, 9, 16))])
def test_pipe16_padded_rows_never_read(emu, config, shape, lds):
    """Padded leading dimensions (odd ones too): the padding holds NaN, so any
    read of it would reach C; the kernel's offsets never touch it, and C's
    padding is never written."""
    M, N, K = shape
    lda, ldb, ldc = lds
    A, B = wl.make_random(M, N, K, seed=K, kind="integer")
    C, errs = run_emu_ld(emu, config, A, B, lda, ldb, ldc)
    assert all(v == 0 for v in errs.values()), errs
    assert np.array_equal(C[:, :N], oracle.gemm_relu(A, B))
    assert np.all(C[:, N:] == 0xFFFF)
