"""The seeded input generator: shapes, dtypes, determinism and value ranges."""
import numpy as np

from tiled_dense_gemm_06_amd import workloads as wl


def test_registry_shapes():
    got = [(wl.WORKLOADS[n].M, wl.WORKLOADS[n].N, wl.WORKLOADS[n].K, wl.WORKLOADS[n].seed) for n in wl.ORDER]
    assert got == [(256, 256, 256, 0), (4096, 4096, 4096, 1), (3001, 2049, 1537, 2),
                   (16, 14336, 4096, 3), (8192, 8192, 8192, 4)]
    w = wl.WORKLOADS["square8192"]
    assert w.flop == 1_099_511_627_776 and w.alg_bytes == 402_653_184
    assert wl.WORKLOADS["skinny16x14336x4096"].alg_bytes == 118_030_336


def test_deterministic_and_typed():
    A1, B1 = wl.make_inputs("square256")
    A2, B2 = wl.make_inputs("square256")
    assert A1.dtype == np.float16 and A1.shape == (256, 256) and A1.flags.c_contiguous
    assert wl.sha256(A1) == wl.sha256(A2) and wl.sha256(B1) == wl.sha256(B2)
    assert wl.sha256(A1) != wl.sha256(B1)


def test_distributions():
    A, B = wl.make_inputs("skinny16x14336x4096")
    assert np.abs(A).max() <= 1.0 and abs(float(A.astype(np.float64).std()) - 1 / np.sqrt(3)) < 0.02
    assert abs(float(B[:512].astype(np.float64).std()) - 0.02) < 0.001
    A, B = wl.make_inputs("ragged3001x2049x1537")
    assert abs(float(A[:256].astype(np.float64).std()) - 1 / np.sqrt(1537)) < 0.001
    Ai, Bi = wl.make_inputs("square256", integer=True)
    assert set(np.unique(Ai).tolist()) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    P, Q = wl.make_random(8, 9, 10, 0, kind="integer_pos")
    assert set(np.unique(P).tolist()) <= {0.0, 1.0, 2.0, 3.0}
