"""GPU parity of the block-scaled (MX) path (tlg_gemm_relu_mx) against the MX
oracle (oracle/oracle_mx.c): bit-exact where every sum is exact in the
hardware's arithmetic (small integer codes, and block scales with small
integers), within a bound derived from that arithmetic otherwise.

The bound. The oracle sums exactly (binary64) and rounds once to fp16. The
kernel's matrix-core step (v_mfma_scale_f32_32x32x64_f8f6f4) adds the
products of each group of 16 consecutive k aligned to the group's largest
product, keeping 13 bits below that product's leading bit (measured on the
device: next to a product of 448, a product of 2^-6 in the same 16-group is
dropped and 2^-5 is kept; in another group both are kept), so a group loses
less than 15 * 2^-13 < 2^-9 of its largest product |p|max(g); groups and
steps are then added in fp32, and C is rounded once to fp16. Hence
|C_gpu - C_ref| <= 2^-10 |C_ref| + 2^-8 G + 2^-24 (K/16 + 64) S + 2^-24,
with G = sum over 16-groups of |p|max(g) (a factor 2 of margin on 2^-9) and
S = sum of all |scaled products|, both from the decoded inputs (torch's own
float8 decoders), scales applied.
"""
import numpy as np
import pytest

import oracle.mx as omx
import tiled_dense_gemm_06_amd as tlg
from test_oracle_mx_pins import ref_decode, unpack
from tiled_dense_gemm_06_amd import _native as nat
from tiled_dense_gemm_06_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FMTS = ["e4m3", "e5m2", "e2m1"]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def bits(t):
    return t.cpu().numpy().view(np.uint16)


def run(fmt, A, SA, Bt, SB, dev, config=-1, out=None):
    C = tlg.gemm_relu_mx(fmt, to_dev(A, dev), to_dev(SA, dev), to_dev(Bt, dev), to_dev(SB, dev), out=out,
                         config=config)
    torch.cuda.synchronize()
    return C


def group_bounds(fmt, A, SA, Bt, SB, rows):
    """(G, S) per output of the given rows: sum over 16-groups of the largest
    |scaled product|, and the sum of all |scaled products|."""
    a = np.abs(ref_decode(fmt, unpack(fmt, A[rows]))) * np.repeat(np.exp2(SA[rows].astype(np.float64) - 127), 32, 1)
    b = np.abs(ref_decode(fmt, unpack(fmt, Bt))) * np.repeat(np.exp2(SB.astype(np.float64) - 127), 32, 1)
    K = a.shape[1]
    G = np.empty((len(rows), b.shape[0]))
    for i in range(len(rows)):
        p = (a[i][None, :] * b).reshape(b.shape[0], K // 16, 16)
        G[i] = p.max(axis=2).sum(axis=1)
    return G, a @ b.T


def assert_mx_close(fmt, got, A, SA, Bt, SB, rows=None, what=""):
    K = A.shape[1] * (2 if fmt == "e2m1" else 1)
    rows = np.arange(A.shape[0]) if rows is None else np.asarray(rows)
    ref = omx.gemm_relu_mx_rows(fmt, A, SA, Bt, SB, rows)
    got = got[rows]
    G, S = group_bounds(fmt, A, SA, Bt, SB, rows)
    g = got.view(np.float16).astype(np.float64)
    r = ref.view(np.float16).astype(np.float64)
    assert np.all(np.isfinite(r)), f"{what}: inputs too large for the bound"
    assert not np.isnan(g).any(), f"{what}: NaN in output"
    tol = 2.0**-10 * np.abs(r) + 2.0**-8 * G + 2.0**-24 * (K / 16 + 64) * S + 2.0**-24
    err = np.abs(g - r)
    bad = err > tol
    worst = float((err / tol).max())
    # for the record: how many elements would also meet the fp16 path's
    # tolerance 1e-2 + 4e-3 |ref| (not the bar here: that tolerance assumes
    # fp16 operands, block-scaled 4- and 8-bit products are summed coarser)
    inside = float((err <= 1e-2 + 4e-3 * np.abs(r)).mean())
    print(f"{what}: max err/bound {worst:.3f}, within 1e-2+4e-3|ref|: {inside:.6f}, max err {err.max():.3g}",
          flush=True)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of bound, max err {err.max()}"
    assert np.all((got & 0x8000) == 0), f"{what}: negative or -0 output"
    return worst


def assert_refused_e2m1_w4(fmt, M, N, K, A, SA, Bt, SB, dev):
    """The four-wave pipelined configuration takes 8-bit codes only: planning
    and a forced call with E2M1 codes must return NOT_SUPPORTED, and the
    forced call must leave C as it was (nothing enqueued)."""
    with pytest.raises(tlg.TlgError) as ei:
        tlg.plan_mx(fmt, M, N, K, config=3)
    assert ei.value.status == nat.TLG_ERROR_NOT_SUPPORTED
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    with pytest.raises(tlg.TlgError) as ei:
        run(fmt, A, SA, Bt, SB, dev, config=3, out=out)
    assert ei.value.status == nat.TLG_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(out).all().item()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("config", [-1, 0, 1, 2, 3])
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 200, 384), (1, 8, 128), (129, 257, 512),
                                   (520, 264, 1152)])
def test_mx_integer_exact(dev, fmt, config, shape):
    """Small integer codes with unit scales: every sum is an exact integer in
    fp32, so the fp16 results must equal the oracle's bit for bit. Ragged M
    and N (several tiles and a partial one), one row, K of 1 to 9 stages."""
    M, N, K = shape
    print(f"mx exact {fmt} config={config} {shape}", flush=True)
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, M, N, K, seed=M + 3 * N + 5 * K, kind="small_int")
    if config == 3 and fmt == "e2m1":
        assert_refused_e2m1_w4(fmt, M, N, K, A, SA, Bt, SB, dev)
        return
    got = bits(run(fmt, A, SA, Bt, SB, dev, config))
    assert np.array_equal(got, omx.gemm_relu_mx(fmt, A, SA, Bt, SB)), (fmt, config, shape)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("config", [-1, 0, 1, 2, 3])
@pytest.mark.parametrize("shape", [(300, 264, 256), (513, 520, 1024), (256, 256, 128), (64, 1000, 2048)])
def test_mx_random_scaled(dev, fmt, config, shape):
    """Random codes over a band of exponents (and zeros/subnormals) with
    random block scales 2^-2 .. 2^2: every element of C within the bound."""
    M, N, K = shape
    print(f"mx random {fmt} config={config} {shape}", flush=True)
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, M, N, K, seed=7 * M + N + K, kind="random")
    if config == 3 and fmt == "e2m1":
        assert_refused_e2m1_w4(fmt, M, N, K, A, SA, Bt, SB, dev)
        return
    got = bits(run(fmt, A, SA, Bt, SB, dev, config))
    worst = assert_mx_close(fmt, got, A, SA, Bt, SB, what=f"{fmt} {config} {shape}")
    assert worst <= 1.0


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_mx_scale_mapping_per_block(dev, fmt):
    """Scales that differ in every block, row and column (2^-4 .. 2^4) with
    small integer codes: every partial sum is a multiple of 2^-8 below 2^14,
    exact in fp32, so the results must equal the oracle's bit for bit; any
    block, row or column scale mixed up in the kernel shows."""
    M, N, K = 130, 136, 256
    A, _, Bt, _ = wl.make_mx_inputs(fmt, M, N, K, seed=3, kind="small_int")
    rng = np.random.default_rng(11)
    SA = rng.integers(123, 132, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(123, 132, size=(N, K // 32)).astype(np.uint8)
    ref = omx.gemm_relu_mx(fmt, A, SA, Bt, SB)
    assert np.all(np.isfinite(ref.view(np.float16)))
    for config in (0, 1, 2) + ((3,) if fmt != "e2m1" else ()):
        got = bits(run(fmt, A, SA, Bt, SB, dev, config))
        assert np.array_equal(got, ref), (fmt, config)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_mx_padded_strides_and_untouched_padding(dev, fmt):
    """Row views with padded leading dimensions for A, B and both scale
    arrays; C is a window of a NaN-filled buffer whose padding must stay NaN."""
    M, N, K = 200, 136, 384
    per = 2 if fmt == "e2m1" else 1
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, M, N, K, seed=21, kind="random")
    Ap = torch.zeros((M, K // per + 32), dtype=torch.uint8, device=dev)
    Bp = torch.zeros((N, K // per + 16), dtype=torch.uint8, device=dev)
    SAp = torch.full((M, K // 32 + 4), 255, dtype=torch.uint8, device=dev)  # padding holds NaN scales
    SBp = torch.full((N, K // 32 + 8), 255, dtype=torch.uint8, device=dev)
    Ap[:, :K // per] = to_dev(A, dev)
    Bp[:, :K // per] = to_dev(Bt, dev)
    SAp[:, :K // 32] = to_dev(SA, dev)
    SBp[:, :K // 32] = to_dev(SB, dev)
    big = torch.full((M + 3, N + 9), float("nan"), dtype=torch.float16, device=dev)
    for config in (0, 1, 2) + ((3,) if fmt != "e2m1" else ()):
        big.fill_(float("nan"))
        tlg.gemm_relu_mx(fmt, Ap[:, :K // per], SAp[:, :K // 32], Bp[:, :K // per], SBp[:, :K // 32],
                         out=big[:M, :N], config=config)
        torch.cuda.synchronize()
        allb = bits(big)
        assert_mx_close(fmt, allb[:M, :N].copy(), A, SA, Bt, SB, what=f"padded {config}")
        assert np.all(np.isnan(allb[:M, N:].view(np.float16))) and np.all(np.isnan(allb[M:].view(np.float16)))


def test_mx_degenerate_and_rejected(dev):
    A, SA, Bt, SB = wl.make_mx_inputs("e4m3", 64, 64, 256, seed=1)
    Ad, SAd, Bd, SBd = (to_dev(x, dev) for x in (A, SA, Bt, SB))
    # K = 0: the empty sum, +0 everywhere
    C = torch.full((5, 7), float("nan"), dtype=torch.float16, device=dev)
    z = torch.zeros((5, 0), dtype=torch.uint8, device=dev)
    tlg.gemm_relu_mx("e4m3", z, z, torch.zeros((7, 0), dtype=torch.uint8, device=dev),
                     torch.zeros((7, 0), dtype=torch.uint8, device=dev), out=C)
    torch.cuda.synchronize()
    assert np.all(bits(C) == 0)
    # M = 0: nothing happens
    out = tlg.gemm_relu_mx("e4m3", Ad[:0], SAd[:0], Bd, SBd)
    assert out.shape == (0, 64)
    # K not a multiple of 32: invalid; a multiple of 32 but not of 128: not supported
    with pytest.raises(tlg.TlgError) as e:
        tlg.gemm_relu_mx("e4m3", Ad[:, :100], SAd[:, :3], Bd[:, :100], SBd[:, :3])
    assert e.value.status == tlg._native.TLG_ERROR_INVALID_VALUE
    with pytest.raises(tlg.TlgError) as e:
        tlg.gemm_relu_mx("e4m3", Ad[:, :96], SAd[:, :3], Bd[:, :96], SBd[:, :3])
    assert e.value.status == tlg._native.TLG_ERROR_NOT_SUPPORTED
    # misaligned A (offset by one byte)
    buf = torch.zeros((64 * 256 + 16,), dtype=torch.uint8, device=dev)
    Amis = buf[1:1 + 64 * 256].view(64, 256)
    with pytest.raises(tlg.TlgError) as e:
        tlg.gemm_relu_mx("e4m3", Amis, SAd, Bd, SBd)
    assert e.value.status == tlg._native.TLG_ERROR_NOT_SUPPORTED


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_mx_square8192_sampled(dev, fmt):
    """The benchmark's workload (8192 cubed, the launch configuration the
    benchmark times): sampled rows against the oracle within the bound."""
    M = N = K = 8192
    print(f"mx square8192 {fmt}", flush=True)
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, M, N, K, seed=4, kind="random")
    assert tlg.plan_mx(fmt, M, N, K)["config_name"] == "mx_256x256_w2x4_s2"
    got = bits(run(fmt, A, SA, Bt, SB, dev))
    rows = np.array([0, 1, 255, 256, 4095, 4096, 8190, 8191] +
                    np.random.default_rng(5).choice(M, 8, replace=False).tolist())
    assert_mx_close(fmt, got, A, SA, Bt, SB, rows=rows, what=f"square8192 {fmt}")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("config", [-1, 0, 1])
def test_mx_grouped(dev, fmt, config):
    """Several block-scaled problems of different shapes (ragged M and N,
    K of 1 to 5 stages, one empty) in one launch: integer codes with block
    scales 2^-4..2^4 (every sum exact in fp32, so bit-exact), each problem
    against the oracle on its own; C prefilled with NaN, padding untouched."""
    shapes = [(300, 264, 256), (1, 8, 128), (129, 520, 640), (0, 64, 128), (256, 256, 384), (70, 33, 128)]
    rng = np.random.default_rng(17)
    probs = []
    for i, (M, N, K) in enumerate(shapes):
        A, _, Bt, _ = wl.make_mx_inputs(fmt, M, N, K, seed=40 + i, kind="small_int")
        SA = rng.integers(123, 132, size=(M, K // 32)).astype(np.uint8)
        SB = rng.integers(123, 132, size=(N, K // 32)).astype(np.uint8)
        probs.append((A, SA, Bt, SB))
    refs = omx.gemm_relu_mx_grouped(fmt, probs)
    bigs = [torch.full((M + 1, N + 8), float("nan"), dtype=torch.float16, device=dev) for M, N, _ in shapes]
    outs = [b[:M, :N] for b, (M, N, _) in zip(bigs, shapes)]
    dev_in = [[to_dev(x, dev) for x in p] for p in probs]
    tlg.gemm_relu_mx_grouped(fmt, *[[p[j] for p in dev_in] for j in range(4)], outs=outs, config=config)
    torch.cuda.synchronize()
    for (M, N, K), b, ref in zip(shapes, bigs, refs):
        allb = bits(b)
        assert np.array_equal(allb[:M, :N], ref), (fmt, config, (M, N, K))
        assert np.all(np.isnan(allb[:M, N:].view(np.float16))) and np.all(np.isnan(allb[M:].view(np.float16)))


def test_mx_grouped_rejects_bad_calls(dev):
    A, SA, Bt, SB = (to_dev(x, dev) for x in wl.make_mx_inputs("e4m3", 64, 64, 256, seed=1))
    with pytest.raises(ValueError):
        tlg.gemm_relu_mx_grouped("e4m3", [A] * 17, [SA] * 17, [Bt] * 17, [SB] * 17)
    with pytest.raises(tlg.TlgError) as e:  # one problem with K % 128 != 0 fails the whole call
        tlg.gemm_relu_mx_grouped("e4m3", [A, A[:, :96]], [SA, SA[:, :3]], [Bt, Bt[:, :96]], [SB, SB[:, :3]])
    assert e.value.status == tlg._native.TLG_ERROR_NOT_SUPPORTED
    assert tlg.gemm_relu_mx_grouped("e4m3", [], [], [], []) == []
    st = tlg._native.tlg_gemm_relu_mx_grouped_variant(tlg.handle_for(dev).ptr, 2, tlg._native.TLG_MX_E4M3, [],
                                                      torch.cuda.current_stream().cuda_stream)
    assert st == tlg._native.TLG_ERROR_INVALID_VALUE
