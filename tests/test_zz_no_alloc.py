"""The allocation-free entry point tlg_gemm_relu_noalloc, through the C ABI,
against tlg_gemm_relu (the handle's entry point) on the same inputs.

Shapes whose plan uses the split kernels' scratch (strips split among
work-groups, with counters and fp32 partials; stream-K over strips) and
shapes that use none. Each pair of calls runs a larger problem and then a
smaller one, back to back on one stream, so the second call finds the
first call's contents in the shared scratch. Bar: bit-exact on
integer-valued inputs (every partial sum is exact in fp32), within
1e-2 + 4e-3 |ref| on uniform inputs; and both against the CPU oracle.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_06_amd as tlg
from tiled_dense_gemm_06_amd import _native as nat
from tiled_dense_gemm_06_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def noalloc(Ad, Bd, Cd, stream):
    M, K = Ad.shape
    N = Bd.shape[1]
    return nat.tlg_gemm_relu_noalloc(M, N, K, Ad.data_ptr(), Ad.stride(0), Bd.data_ptr(), Bd.stride(0),
                                     Cd.data_ptr(), Cd.stride(0), stream.cuda_stream)


def close(got, ref):
    g = got.view(np.float16).astype(np.float64)
    r = ref.view(np.float16).astype(np.float64)
    return bool(np.all(np.abs(g - r) <= 1e-2 + 4e-3 * np.abs(r)) and not np.isnan(g).any())


PAIRS = [
    ((1, 4096, 4096), (1, 2048, 1024)),        # strips split in 4 parts, then in 4 parts on fewer strips
    ((8, 8192, 8192), (4, 2048, 2048)),        # stream-K strips, then split strips
    ((48, 4096, 14336), (40, 264, 4096)),      # 64-row strips in 4 parts, then 5 strips in 4 parts
    ((16, 14336, 4096), (16, 2048, 4096)),     # whole strips (no scratch), then split strips
    ((512, 512, 264), (200, 264, 520)),        # tiles (no scratch)
]


@pytest.mark.parametrize("kind", ["integer", "uniform"])
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "%dx%dx%d_then_%dx%dx%d" % (p[0] + p[1]))
def test_noalloc_matches_handle_entry_point(dev, pair, kind):
    assert nat.tlg_noalloc_scratch_bytes() == (64 << 10) + (8 << 20)
    stream = torch.cuda.current_stream(dev)
    outs, refs = [], []
    for shape in pair:
        M, N, K = shape
        print(f"noalloc {shape} {kind} plan={tlg.plan(M, N, K)['config_name']}", flush=True)
        A, B = wl.make_random(M, N, K, seed=M + 7 * N + 3 * K, kind=kind)
        Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
        Cn = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
        st = noalloc(Ad, Bd, Cn, stream)
        assert st == nat.TLG_SUCCESS, nat.tlg_status_string(st)
        outs.append((Ad, Bd, Cn, A, B))
    torch.cuda.synchronize()
    for Ad, Bd, Cn, A, B in outs:
        Ch = tlg.gemm_relu(Ad, Bd)  # the handle's entry point on the same inputs
        torch.cuda.synchronize()
        got = Cn.cpu().numpy().view(np.uint16)
        ref_h = Ch.cpu().numpy().view(np.uint16)
        ref_o = oracle.gemm_relu(A, B)
        if kind == "integer":
            assert np.array_equal(got, ref_h), A.shape
            assert np.array_equal(got, ref_o), A.shape
        else:
            assert close(got, ref_h) and close(got, ref_o), A.shape


def test_noalloc_argument_errors(dev):
    """The same argument checks as tlg_gemm_relu; nothing is enqueued."""
    stream = torch.cuda.current_stream(dev)
    C = torch.full((4, 8), float("nan"), dtype=torch.float16, device=dev)
    A = torch.zeros((4, 8), dtype=torch.float16, device=dev)
    B = torch.zeros((8, 8), dtype=torch.float16, device=dev)
    s = stream.cuda_stream
    assert nat.tlg_gemm_relu_noalloc(-1, 8, 8, A.data_ptr(), 8, B.data_ptr(), 8, C.data_ptr(), 8, s) == 1
    assert nat.tlg_gemm_relu_noalloc(4, 8, 8, A.data_ptr(), 7, B.data_ptr(), 8, C.data_ptr(), 8, s) == 1
    assert nat.tlg_gemm_relu_noalloc(4, 8, 8, 0, 8, B.data_ptr(), 8, C.data_ptr(), 8, s) == 1
    assert nat.tlg_gemm_relu_noalloc(0, 8, 8, 0, 8, 0, 8, 0, 8, s) == 0
    torch.cuda.synchronize()
    assert torch.isnan(C).all().item()
    # K == 0: C becomes +0 everywhere
    assert nat.tlg_gemm_relu_noalloc(4, 8, 0, A.data_ptr(), 1, B.data_ptr(), 8, C.data_ptr(), 8, s) == 0
    torch.cuda.synchronize()
    assert (C.cpu().numpy().view(np.uint16) == 0).all()
