"""The C-ABI library without a GPU: it loads, exports every entry point that
include/tlg.h declares, and its pure host logic (argument checks, kernel
choice, architecture check, status strings) behaves as documented."""
import ctypes
import os
import re

import pytest

import tiled_dense_gemm_06_amd as tlg
from tiled_dense_gemm_06_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tlg.h")

A16 = 1 << 20  # stand-in device addresses (never dereferenced on the host)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tlg_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "tlg_gemm_relu" in names and "tlg_create" in names and "tlg_destroy" in names
    L = ctypes.CDLL(nat.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert tlg.tlg_version() >= 100
    for st in range(5):
        assert tlg.tlg_status_string(st).startswith("TLG_")
    assert "unknown" in tlg.tlg_status_string(99)


def test_arch_check():
    assert tlg.tlg_arch_supported("gfx950")
    assert tlg.tlg_arch_supported("gfx950:sramecc+:xnack-")
    for bad in ["gfx942", "gfx9500", "gfx90a", "", "sm_90", "gfx95"]:
        assert not tlg.tlg_arch_supported(bad), bad


@pytest.mark.parametrize("args,expect", [
    ((4, 4, 4, A16, 4, A16, 4, A16, 4), 0),
    ((-1, 4, 4, A16, 4, A16, 4, A16, 4), 1),
    ((4, -1, 4, A16, 4, A16, 4, A16, 4), 1),
    ((4, 4, -1, A16, 4, A16, 4, A16, 4), 1),
    ((4, 4, 4, A16, 3, A16, 4, A16, 4), 1),   # lda < K
    ((4, 4, 4, A16, 4, A16, 3, A16, 4), 1),   # ldb < N
    ((4, 4, 4, A16, 4, A16, 4, A16, 3), 1),   # ldc < N
    ((4, 4, 4, 0, 4, A16, 4, A16, 4), 1),     # A NULL
    ((4, 4, 4, A16, 4, 0, 4, A16, 4), 1),     # B NULL
    ((4, 4, 4, A16, 4, A16, 4, 0, 4), 1),     # C NULL
    ((4, 4, 4, A16 + 1, 4, A16, 4, A16, 4), 1),  # odd address
    ((0, 4, 4, 0, 4, 0, 4, 0, 4), 0),         # M == 0: nothing touched, NULLs allowed
    ((4, 0, 4, 0, 4, 0, 1, 0, 1), 0),         # N == 0
    ((4, 4, 0, 0, 1, 0, 4, A16, 4), 0),       # K == 0: A and B unused, C needed
    ((4, 4, 0, 0, 1, 0, 4, 0, 4), 1),         # K == 0 but C NULL
])
def test_check_args(args, expect):
    assert tlg.tlg_check_args(*args) == expect


def test_plan_shapes_of_the_workloads():
    # K a multiple of 64 and N of 8: the 16 x 16 x 32 MFMA tiles
    assert tlg.plan(8192, 8192, 8192)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"
    assert tlg.plan(4096, 4096, 4096)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"
    # and for any K from 256 tiles of 256 x 256 up
    assert tlg.plan(4096, 4096, 4104)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"
    assert tlg.plan(8192, 8192, 8200)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"
    # otherwise the eight-wave 32 x 32 x 16 tiles: a K tail below 256 tiles,
    # N not a multiple of 8
    assert tlg.plan(3072, 3072, 3080)["config_name"] == "pipe_256x256x64_w2x4_s2_a3_early"
    # tile height by rounds x relative tile time: 272 tiles of 256 x 256 take
    # two rounds, 374 of 192 x 256 two cheaper ones; 576 and 768 take three
    # each; 400 of 256 x 256 two rounds against three of 192 x 256
    assert tlg.plan(4096, 4104, 4096)["config_name"] == "pipe16_192x256x64_w2x2_s2_a3_sp6"
    assert tlg.plan(6144, 6144, 6144)["config_name"] == "pipe16_192x256x64_w2x2_s2_a3_sp6"
    assert tlg.plan(5120, 5120, 5120)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"
    assert tlg.plan(4096, 4100, 4096, aligned=True, ldb=4104, ldc=4104)["config_name"] == \
        "pipe_256x256x64_w2x4_s2_a3_early"
    # B transposed from 128 tiles of 256 x 256: the 16 x 16 x 32 tiles under
    # the plain call's conditions, else the 32 x 32 x 16 early ones
    assert tlg.plan(8192, 8192, 8192, trans_b=True)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"
    assert tlg.plan(4096, 4096, 4104, trans_b=True)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"
    assert tlg.plan(3072, 3072, 3080, trans_b=True)["config_name"] == "pipe_256x256x64_w2x4_s2_a3_early"
    assert tlg.plan(4096, 4352, 4104, trans_b=True)["config_name"] == "pipe_256x256x64_w2x4_s2_a3_early"
    # skinny M with B transposed: the strip kernel under the plain call's rule
    for shape, name, parts in (((16, 14336, 4096), "splitk_waves_32x64x64_w2_s3", 1),
                               ((1, 4096, 4096), "splitk_waves_32x64x64_w2_s3", 4),
                               ((48, 4096, 14336), "splitk_waves_64x64x64_w2_s3", 4)):
        info = tlg.plan(*shape, trans_b=True)
        assert (info["config_name"], info["splits"]) == (name, parts), shape
        assert info["config_name"] == tlg.plan(*shape)["config_name"], shape
    assert tlg.plan(16, 14336, 256, trans_b=True)["variant_name"] == "tiled_dma"  # K below 512
    assert tlg.plan(16, 14336, 4096, trans_b=True, ldb=4100)["variant_name"] == "tiled_dma"  # ldb % 8
    with pytest.raises(tlg.TlgError):
        tlg.plan(100, 4096, 4096, variant=tlg.TLG_VARIANT_SPLITK, config=3, trans_b=True)  # M above the strip
    with pytest.raises(tlg.TlgError):
        tlg.plan(16, 4096, 4096, variant=tlg.TLG_VARIANT_SPLITK, config=0, trans_b=True)  # not a strip
    # ... and the plain call's tile height by rounds (K whole stages)
    assert tlg.plan(3072, 3072, 3072, trans_b=True)["config_name"] == "pipe16_192x256x64_w2x2_s2_a3_sp6"
    assert tlg.plan(2048, 4096, 4096, trans_b=True)["config_name"] == "pipe16_128x256x64_w1x4_s3_a3"
    for shape in ((3072, 3072, 3072), (6144, 6144, 6144), (2560, 4096, 4096), (2048, 4096, 4096), (8192, 8192, 8192),
                  (4096, 4352, 4096)):
        assert tlg.plan(*shape, trans_b=True)["config_name"] == tlg.plan(*shape)["config_name"], shape
    # B transposed below 128 tiles of 256 x 256: 128 x 256 pipelined tiles
    # from 192 of them, else the direct-to-LDS tiles by count
    assert tlg.plan(3001, 2049, 1537, trans_b=True)["config_name"] == "pipe16_128x256x64_w1x4_s3_a3"
    assert tlg.plan(2560, 2560, 2560, trans_b=True)["config_name"] == "pipe16_128x256x64_w1x4_s3_a3"
    assert tlg.plan(2048, 2048, 2048, trans_b=True)["config_name"] == "dma_128x128x32_w2x2_s4"
    # odd sizes and leading dimensions: direct-to-LDS loads, staged K tail; the
    # tuned table gives this class the pipelined 128 x 256 tiles (216 of them)
    p = tlg.plan(3001, 2049, 1537)
    assert p["variant_name"] == "tiled_pipe" and p["config_name"] == "pipe_128x256x64_w1x4_s3" and p["grid"] == 216
    # the same shape without the table's entry: the heuristic's 128 x 128 tiles
    p = tlg.plan(3001, 2049, 1537, variant=tlg.TLG_VARIANT_TILED_DMA)
    assert p["config_name"] == "dma_128x128x32_w2x2_s4"
    p = tlg.plan(16, 14336, 4096)  # one work-group per 64 columns, K split among its waves
    assert p["variant_name"] == "splitk" and p["config_name"] == "splitk_waves_32x64x64_w2_s3"
    assert p["kernels"] == 1 and p["grid"] == 14336 // 64 and p["workspace_bytes"] == 0
    p = tlg.plan(16, 14336, 4096, variant=tlg.TLG_VARIANT_SPLITK, config=2)  # stream-K
    assert p["config_name"].startswith("streamk") and p["kernels"] == 1
    assert p["grid"] == 2 * 256 and p["splits"] >= 2  # two work-groups per CU, ~4.6 per output tile
    assert p["workspace_bytes"] == (64 << 10) + p["grid"] * 2 * 32 * 128 * 4 <= tlg.tlg_workspace_bytes()
    # 32 < M <= 64, aligned: 64-row strips from K = 2048 up, tiles below
    assert tlg.plan(48, 14336, 4096)["config_name"] == "splitk_waves_64x64x64_w2_s3"
    assert tlg.plan(48, 4096, 4096)["config_name"] == "splitk_waves_64x64x64_w2_s3"
    assert tlg.plan(64, 1024, 2048)["config_name"] == "splitk_waves_64x64x64_w2_s3"
    assert tlg.plan(48, 4096, 1024)["variant_name"] == "tiled_dma"
    # M > 64: no strips; with K >= 4096 and fewer 64 x 64 tiles than CUs, K
    # split over 32 x 128 tiles and a second kernel's ordered sum
    p = tlg.plan(65, 4096, 4096)
    assert p["config_name"] == "splitk_32x128x64_w1x4_s4" and p["kernels"] == 2 and p["splits"] == 6
    assert tlg.plan(65, 4096, 2048)["variant_name"] == "tiled_dma"
    for shape, splits in [((512, 512, 4096), 4), ((1024, 512, 4096), 4), ((1024, 1024, 8192), 2),
                          ((256, 256, 16384), 16)]:
        p = tlg.plan(*shape)
        assert p["config_name"] == "splitk_32x128x64_w1x4_s4" and p["splits"] == splits, shape
        assert p["workspace_bytes"] == (64 << 10) + splits * shape[0] * shape[1] * 4 <= tlg.tlg_workspace_bytes()
    assert tlg.plan(1024, 1024, 4096)["variant_name"] == "tiled_dma"  # a full round of 64 x 64 tiles
    assert tlg.plan(512, 512, 4096, lda=4100)["variant_name"] == "tiled_dma"  # unaligned rows: no split
    # fewer than 128 tiles of 256 x 256: the 32 x 32 x 16 128 x 256 tiles from 96 of them up
    for shape, grid in [((2048, 2048, 2048), 128), ((1536, 2048, 4096), 96), ((2048, 2048, 8192), 128)]:
        p = tlg.plan(*shape)
        assert p["config_name"] == "pipe_128x256x64_w1x4_s3" and p["grid"] == grid, shape
    assert tlg.plan(1280, 2048, 2048)["variant_name"] == "tiled_dma"  # 80 of them
    # unaligned (the split-K kernels load 16-byte pieces): tiles
    assert tlg.plan(48, 4100, 4096)["variant_name"] == "tiled_dma"
    p = tlg.plan(16, 2048, 4096)  # few strips: K split among work-groups too, up to the CUs
    assert p["config_name"] == "splitk_waves_32x64x64_w2_s3" and p["splits"] == 4 and p["grid"] == 32 * 4
    p = tlg.plan(1, 4096, 4096)
    assert p["config_name"] == "splitk_waves_32x64x64_w2_s3" and p["splits"] == 4 and p["grid"] == 64 * 4
    # fewer than 256 tiles of 256 x 256: 129-256 tiles of 128 x 256, else
    # 192 x 256 tiles while they fit one wave, else 256 x 256
    p = tlg.plan(3072, 3072, 3072)  # 144 tiles of 256 x 256, 288 of 128 x 256, 192 of 192 x 256
    assert p["config_name"] == "pipe16_192x256x64_w2x2_s2_a3_sp6" and p["grid"] == 192
    p = tlg.plan(2560, 2560, 2560)  # 200 tiles of 128 x 256
    assert p["config_name"] == "pipe16_128x256x64_w1x4_s3_a3" and p["grid"] == 200
    p = tlg.plan(2560, 2560, 2568)  # a K tail: the 32 x 32 x 16 half tiles
    assert p["config_name"] == "pipe_128x256x64_w1x4_s3" and p["grid"] == 200
    assert tlg.plan(8192, 1024, 4096)["config_name"] == "pipe16_128x256x64_w1x4_s3_a3"  # 256 tiles of 128 x 256
    assert tlg.plan(4096, 3072, 4096)["config_name"] == "pipe16_256x256x64_w2x2_s2_a3_sp8"  # 264 of 192 x 256
    # 128 tiles of 128 x 256: the 32 x 32 x 16 form
    assert tlg.plan(2048, 2048, 2048)["config_name"] == "pipe_128x256x64_w1x4_s3"
    # forced 16 x 16 x 32 tiles take any K and N (whole stages, then a masked
    # stage and a zero-padded block); with B transposed only the three
    # pipelined ones (17, 21, 26) are built
    assert tlg.plan(300, 264, 200, variant=tlg.TLG_VARIANT_TILED_PIPE, config=10)["config_name"] == \
        "pipe16_256x256x64_w2x2_s2_a3"
    assert tlg.plan(300, 260, 256, variant=tlg.TLG_VARIANT_TILED_PIPE, config=10, ldb=264, ldc=264)["grid"] == 4
    with pytest.raises(tlg.TlgError):
        tlg.plan(512, 512, 512, variant=tlg.TLG_VARIANT_TILED_PIPE, config=10, trans_b=True)
    for cfg, bm in ((17, 256), (21, 128), (26, 192)):
        info = tlg.plan(1000, 1000, 200, variant=tlg.TLG_VARIANT_TILED_PIPE, config=cfg, trans_b=True)
        assert info["grid"] == -(-1000 // bm) * 4, (cfg, info)
    assert tlg.plan(256, 256, 256)["variant_name"] == "tiled_dma"
    assert tlg.plan(5, 7, 0)["variant_name"] == "fill_zero"
    assert tlg.plan(0, 7, 9)["variant_name"] == "noop"
    assert tlg.plan(7, 0, 9)["variant_name"] == "noop"


def test_plan_alignment_and_edges():
    # the tiled direct-to-LDS kernels take any 2-byte aligned data
    for kw in [dict(aligned=False), dict(lda=520), dict(lda=513), {}, dict(ldc=515)]:
        assert tlg.plan(512, 512, 512, **kw)["variant_name"] == "tiled_dma", kw
    assert tlg.plan(512, 516, 512)["variant_name"] == "tiled_dma"  # N % 8 != 0
    assert tlg.plan(512, 512, 500)["variant_name"] == "tiled_dma"  # K % 8 != 0
    # a chunk crossing the N edge must stay inside the next row of B
    assert tlg.plan(512, 5, 512)["variant_name"] == "tiled_general"
    assert tlg.plan(512, 5, 512, ldb=8)["variant_name"] == "tiled_dma"
    # the skinny kernels need aligned data
    assert tlg.plan(16, 14336, 4096)["variant_name"] == "splitk"
    assert tlg.plan(16, 14336, 4096, aligned=False)["variant_name"] != "splitk"
    assert tlg.plan(16, 14336, 4095)["variant_name"] != "splitk"


def test_forced_variants():
    with pytest.raises(tlg.TlgError):  # chunks crossing N would leave the next row of B
        tlg.plan(512, 5, 512, variant=tlg.TLG_VARIANT_TILED_DMA)
    assert tlg.plan(512, 512, 512, aligned=False, variant=tlg.TLG_VARIANT_TILED_DMA)["variant_name"] == "tiled_dma"
    with pytest.raises(tlg.TlgError):
        tlg.plan(16, 14336, 4095, variant=tlg.TLG_VARIANT_SPLITK)
    p = tlg.plan(16, 14336, 4096, variant=tlg.TLG_VARIANT_SPLITK, config=0, splits=8)
    assert p["splits"] == 8 and p["grid"] == 112 * 8 and p["kernels"] == 2
    p = tlg.plan(16, 256, 64, variant=tlg.TLG_VARIANT_SPLITK, config=2)  # stream-K: never more work-groups
    assert p["grid"] == 2 * 1 and p["kernels"] == 1                         # than iterations
    p = tlg.plan(16, 256, 64, variant=tlg.TLG_VARIANT_SPLITK)  # strips: never more parts than K blocks
    assert p["config_name"] == "splitk_waves_32x64x64_w2_s3" and p["grid"] == 4 and p["splits"] == 1
    p = tlg.plan(300, 300, 300, variant=tlg.TLG_VARIANT_NAIVE)
    assert p["variant_name"] == "naive"
    p = tlg.plan(300, 304, 304, variant=tlg.TLG_VARIANT_TILED_GENERAL)
    assert p["variant_name"] == "tiled_general"
    p = tlg.plan(300, 304, 304, variant=tlg.TLG_VARIANT_TILED_PIPE)  # forced: any shape
    assert p["variant_name"] == "tiled_pipe" and p["grid"] == 2 * 2
    p = tlg.plan(300, 300, 301, aligned=False, variant=tlg.TLG_VARIANT_TILED_PIPE)
    assert p["variant_name"] == "tiled_pipe"
    with pytest.raises(tlg.TlgError):
        tlg.plan(300, 7, 300, variant=tlg.TLG_VARIANT_TILED_PIPE)  # ldb < 8 with N % 8 != 0
    with pytest.raises(tlg.TlgError):
        tlg.plan(4, 4, 4, variant=99)
    with pytest.raises(tlg.TlgError):  # a configuration needs a forced variant
        tlg.plan(512, 512, 512, config=0)
    with pytest.raises(tlg.TlgError):  # no such configuration
        tlg.plan(512, 512, 512, variant=tlg.TLG_VARIANT_TILED_PIPE, config=99)
    for cfg in range(5):
        p = tlg.plan(1024, 1024, 1024, variant=tlg.TLG_VARIANT_TILED_PIPE, config=cfg)
        assert p["config"] == cfg and p["config_name"].startswith("pipe_256x256")


def test_split_counts_cover_k_without_empty_splits():
    for K in [512, 520, 1000, 4096, 4104, 8192, 65536]:
        for forced in [0, 2, 3, 7, 16, 64]:
            try:
                p = tlg.plan(16, 1024, K - K % 8, variant=tlg.TLG_VARIANT_SPLITK, config=0, splits=forced)
            except tlg.TlgError:
                continue
            s, bk = p["splits"], p["block_k"]
            k = K - K % 8
            ksteps = -(-k // bk)
            k_split = -(-ksteps // s) * bk
            assert (s - 1) * k_split < k <= s * k_split, (K, forced, s)


def test_workspace_cap_lowers_splits():
    cap = (64 << 10) + 2 * 64 * 14336 * 4
    st, info = nat.tlg_plan(64, 14336, 4096, A16, 4096, A16, 14336, A16, 14336, tlg.TLG_VARIANT_SPLITK, 0, 16, cap)
    assert st == 0 and info.splits <= 2 and info.workspace_bytes <= cap
    cap = (64 << 10) + 100 * 2 * 32 * 128 * 4  # stream-K: the grid shrinks to fit its partial slots
    st, info = nat.tlg_plan(64, 14336, 4096, A16, 4096, A16, 14336, A16, 14336, tlg.TLG_VARIANT_SPLITK, 2, 0, cap)
    assert st == 0 and info.grid == 100 and info.workspace_bytes == cap


def test_gemm_relu_rejects_null_handle():
    # no GPU needed: the handle check comes first
    st = nat.tlg_gemm_relu(None, 4, 4, 4, A16, 4, A16, 4, A16, 4, None)
    assert st == nat.TLG_ERROR_INVALID_VALUE
    assert nat.tlg_destroy(None) == 0


_TABLE = os.path.join(os.path.dirname(tlg.__file__), "csrc", "tune_table.inc")
_ENTRY = re.compile(r"^\s*\{(-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+)\},\s*//\s*(\d+)x(\d+)x(\d+):")


def _tune_entries():
    out = []
    with open(_TABLE) as f:
        for line in f:
            m = _ENTRY.match(line)
            if m:
                v = [int(x) for x in m.groups()]
                out.append((tuple(v[:7]), tuple(v[7:])))
    return out


def _clog2(x):
    return 0 if x <= 1 else (x - 1).bit_length()


def test_tuned_table_entries_are_taken():
    """Every measured entry of the compiled-in table decides the plan of its
    own shape (the class key matches the shape), and an entry the problem
    cannot take (unaligned pointers for a direct-to-LDS kernel) falls back to
    the heuristic instead of failing."""
    entries = _tune_entries()
    for (lm, ln, lk, rg, variant, config, splits), (M, N, K) in entries:
        assert (lm, ln, lk, rg) == (_clog2(M), _clog2(N), _clog2(K), 1 if (K % 8 or N % 8) else 0)
        p = tlg.plan(M, N, K)
        assert (p["variant"], p["config"]) == (variant, config), (M, N, K, p)
        if splits:
            assert p["splits"] == splits
        forced = tlg.plan(M, N, K, variant=variant, config=config, splits=splits)
        assert (forced["grid"], forced["splits"]) == (p["grid"], p["splits"])
        q = tlg.plan(M, N, K, aligned=False)
        if variant == tlg.TLG_VARIANT_SPLITK:  # split-K kernels need 16-byte aligned data: the heuristic
            assert q["variant_name"] in ("tiled_dma", "tiled_general")
        else:  # the direct-to-LDS tile kernels load unaligned rows too
            assert (q["variant"], q["config"]) == (variant, config)


def test_tuned_classes_of_the_table():
    # the two measured skinny classes with 32 < M <= 64: 64-row strips (B read once)
    assert tlg.plan(48, 4096, 14336)["config_name"] == "splitk_waves_64x64x64_w2_s3"
    assert tlg.plan(64, 4096, 8192)["config_name"] == "splitk_waves_64x64x64_w2_s3"
    # mid-size and ragged classes: pipelined 128 x 256 tiles; decode-like
    # 8 x 8192 x 8192: stream-K over strips
    assert tlg.plan(1024, 4096, 16384)["config_name"] == "pipe_128x256x64_w1x4_s3"
    assert tlg.plan(3001, 2049, 1537)["config_name"] == "pipe_128x256x64_w1x4_s3"
    p = tlg.plan(8, 8192, 8192)
    assert p["config_name"] == "strip_sk_32x64x64_w2_s3" and p["grid"] == 256
    # a neighbouring class (shorter K) keeps the heuristic's choice
    assert tlg.plan(48, 4096, 1024)["variant_name"] == "tiled_dma"


def test_plan_block_scaled():
    p = tlg.plan_mx("e4m3", 8192, 8192, 8192)
    assert p["config_name"] == "mx_256x256_w2x4_s2" and p["grid"] == 32 * 32 and p["block_k"] == 128
    p = tlg.plan_mx("e2m1", 8192, 8192, 8192)
    assert p["config_name"] == "mx_256x256_w2x4_s2" and p["block_k"] == 256  # 4-bit codes: 256 per stage
    p = tlg.plan_mx("e5m2", 300, 200, 384)
    assert p["config_name"] == "mx_128x128_w2x2_s3" and p["grid"] == 3 * 2 and p["threads"] == 256
    assert tlg.plan_mx("e4m3", 300, 200, 384, config=0)["grid"] == 2 * 1
    assert tlg.plan_mx("e4m3", 0, 5, 128)["variant_name"] == "noop"
    assert tlg.plan_mx("e4m3", 5, 5, 0)["variant_name"] == "fill_zero"
    S, NS, INV = tlg.TlgError, nat.TLG_ERROR_NOT_SUPPORTED, nat.TLG_ERROR_INVALID_VALUE
    cases = [
        (dict(fmt="e4m3", M=64, N=64, K=100), INV),              # K not whole blocks of 32
        (dict(fmt="e4m3", M=64, N=64, K=96), NS),                # K not a multiple of 128
        (dict(fmt="e4m3", M=64, N=64, K=256, aligned=False), NS),
        (dict(fmt="e4m3", M=64, N=64, K=256, lda=264), NS),      # rows not a multiple of 16 bytes
        (dict(fmt="e2m1", M=64, N=64, K=256, lda=264), NS),      # 132-byte rows
        (dict(fmt="e2m1", M=64, N=64, K=256, lda=257), INV),     # packed codes: even leading dimension
        (dict(fmt="e4m3", M=64, N=64, K=256, ldsa=9), NS),       # scale rows not whole dwords
        (dict(fmt="e4m3", M=64, N=64, K=256, ldsb=7), INV),      # scale rows shorter than K/32
        (dict(fmt="e4m3", M=64, N=64, K=256, lda=128), INV),     # lda < K
        (dict(fmt="e4m3", M=64, N=64, K=256, config=4), INV),
        (dict(fmt="e2m1", M=64, N=64, K=256, config=3), NS),        # four-wave pipelined: 8-bit only
    ]
    for kw, status in cases:
        kw = dict(kw)
        fmt, M, N, K = kw.pop("fmt"), kw.pop("M"), kw.pop("N"), kw.pop("K")
        with pytest.raises(S) as e:
            tlg.plan_mx(fmt, M, N, K, **kw)
        assert e.value.status == status, (fmt, M, N, K, kw)
    with pytest.raises(ValueError):
        tlg.plan_mx("e3m2", 64, 64, 256)
    st, _ = nat.tlg_plan_mx(7, 64, 64, 256, 1 << 20, 256, 1 << 20, 8, 1 << 20, 256, 1 << 20, 8, 1 << 20, 64)
    assert st == INV
    assert nat.tlg_plan_mx_config_name(0) == "mx_256x256_w2x4_s2" and nat.tlg_plan_mx_config_name(4) == ""


def test_plan_pingpong_forced_only():
    p = tlg.plan(8192, 8192, 8192, variant=tlg.TLG_VARIANT_PINGPONG)
    assert p["variant_name"] == "pingpong" and p["config_name"] == "pingpong_256x256x32_w2x4_s4"
    assert p["grid"] == 32 * 32 and p["threads"] == 512 and p["block_k"] == 32
    assert tlg.plan(8192, 8192, 8192)["variant_name"] == "tiled_pipe"  # not the default
    assert tlg.plan(301, 259, 203, variant=tlg.TLG_VARIANT_PINGPONG, trans_b=True)["grid"] == 2 * 2
    assert tlg.plan(300, 300, 301, aligned=False, variant=tlg.TLG_VARIANT_PINGPONG)["grid"] == 4
    with pytest.raises(tlg.TlgError):
        tlg.plan(300, 7, 300, variant=tlg.TLG_VARIANT_PINGPONG)  # ldb < 8 with N % 8 != 0
    with pytest.raises(tlg.TlgError):
        tlg.plan(512, 512, 512, variant=tlg.TLG_VARIANT_PINGPONG, config=1)
    assert tlg.tlg_plan_config_name(tlg.TLG_VARIANT_PINGPONG, 0) == "pingpong_256x256x32_w2x4_s4"
    with pytest.raises(tlg.TlgError):
        tlg.plan(64, 64, 64, variant=tlg.TLG_VARIANT_PINGPONG + 1)


def test_strip_configurations_plan():
    """Every strip configuration of the split-K family (forced): its name,
    its strips x parts grid for 16 x 14336 x 4096 (224 64-column, 112
    128-column, 56 256-column strips, parts filling the CUs), the partial
    workspace of split strips; the stream-K strips take one range per CU
    (two for the two-stage form) and need at least one range per strip; M
    above one strip is refused."""
    V = tlg.TLG_VARIANT_SPLITK
    want = {3: ("splitk_waves_32x64x64_w2_s3", 224, 1), 4: ("splitk_waves_32x64x64_w4_s3", 224, 1),
            5: ("splitk_waves_32x64x64_w2_s4", 224, 1), 6: ("splitk_waves_32x128x64_w2_s3", 224, 2),
            7: ("splitk_waves_32x128x64_w4_s2", 224, 2), 8: ("splitk_waves_32x256x32_w2_s3", 224, 4),
            9: ("splitk_waves_64x64x64_w2_s3", 224, 1),
            10: ("strip_sk_32x64x64_w2_s3", 256, None), 11: ("strip_sk_32x64x64_w2_s2", 512, None)}
    for c, (name, grid, parts) in want.items():
        p = tlg.plan(16, 14336, 4096, variant=V, config=c)
        assert (p["config_name"], p["grid"]) == (name, grid), c
        assert tlg.tlg_plan_config_name(V, c) == name
        if parts is not None:
            assert p["splits"] == parts
            bn = p["block_n"]
            bm = p["block_m"]
            assert p["workspace_bytes"] == (0 if parts == 1 else (64 << 10) + (14336 // bn) * parts * bm * bn * 4)
        else:  # two partial slots per range
            assert p["workspace_bytes"] == (64 << 10) + grid * 2 * 32 * 64 * 4
    for c in want:  # M above the strip's rows
        with pytest.raises(tlg.TlgError):
            tlg.plan(65 if c == 9 else 48, 14336, 4096, variant=V, config=c)
    # the 64-row strip: 48 x 4096 x 14336 in 64 strips of 4 parts, B read once
    p = tlg.plan(48, 4096, 14336, variant=V, config=9)
    assert (p["block_m"], p["grid"], p["splits"]) == (64, 256, 4)
    assert p["workspace_bytes"] == (64 << 10) + 64 * 4 * 64 * 64 * 4
    with pytest.raises(tlg.TlgError):  # 300 strips, 256 ranges: a range would cross three strips
        tlg.plan(16, 64 * 300, 4096, variant=V, config=10)
    assert tlg.plan(16, 64 * 300, 4096, variant=V, config=11)["grid"] == 512
    with pytest.raises(tlg.TlgError):
        tlg.plan(16, 14336, 4096, variant=V, config=12)


def test_zero_k_plans_of_every_call_refuse_sizes_beyond_the_limit():
    """K == 0 plans the fill kernel (256 threads, at most 65536 work-groups);
    sizes beyond the library's limit are refused before M * N is formed, in
    the plain, transposed-B and block-scaled planners alike."""
    big = (1 << 40)
    for M, N in ((big, 8), (8, big), ((1 << 31) - 1024 + 1, 1)):
        st, _ = nat.tlg_plan(M, N, 0, A16, 1, A16, N, A16, N)
        assert st == nat.TLG_ERROR_NOT_SUPPORTED, (M, N)
        st, _ = nat.tlg_plan_bt(M, N, 0, A16, 1, A16, 1, A16, N, 0, -1)
        assert st == nat.TLG_ERROR_NOT_SUPPORTED, (M, N)
        with pytest.raises(tlg.TlgError):
            tlg.plan_mx("e4m3", M, N, 0)
    for f in (lambda: tlg.plan(5, 7, 0), lambda: tlg.plan(5, 7, 0, trans_b=True),
              lambda: tlg.plan_mx("e4m3", 5, 7, 0)):
        p = f()
        assert p["variant_name"] == "fill_zero" and p["threads"] == 256 and p["grid"] == 1
    assert tlg.plan(4096, 4096, 0)["grid"] == 65536


def test_streamk_plan_of_huge_forced_shapes_does_not_overflow():
    """Forced stream-K on sizes with more tiles than counters: refused, and
    the iteration count is never formed from a tile count that large."""
    st, _ = nat.tlg_plan(1 << 30, 1 << 24, 1 << 25, A16, 1 << 25, A16, 1 << 24, A16, 1 << 24,
                         tlg.TLG_VARIANT_SPLITK, 2, 0)
    assert st == nat.TLG_ERROR_NOT_SUPPORTED


def test_status_string_of_any_int():
    L = ctypes.CDLL(nat.LIB_PATH)
    L.tlg_status_string.argtypes = [ctypes.c_int]
    L.tlg_status_string.restype = ctypes.c_char_p
    for v in (-2, -1, 5, 7, 1 << 20):
        assert L.tlg_status_string(v) == b"unknown tlg_status"


def test_noalloc_entry_point_checks_arguments_without_a_gpu():
    """tlg_gemm_relu_noalloc checks its arguments as tlg_gemm_relu does,
    before any device call: bad arguments give TLG_ERROR_INVALID_VALUE."""
    assert nat.tlg_noalloc_scratch_bytes() == (64 << 10) + (8 << 20)
    bad = [(-1, 4, 4, A16, 4, A16, 4, A16, 4), (4, 4, 4, A16, 3, A16, 4, A16, 4), (4, 4, 4, 0, 4, A16, 4, A16, 4),
           (4, 4, 4, A16 + 1, 4, A16, 4, A16, 4), (4, 4, 4, A16, 4, A16, 4, A16, 3)]
    for args in bad:
        assert nat.tlg_gemm_relu_noalloc(*args, 0) == nat.TLG_ERROR_INVALID_VALUE, args


def test_grids_beyond_int32_are_refused():
    """Every kernel computes its tile indices in 32-bit integers, so a plan
    that would need more than INT32_MAX work-groups is refused (only an
    output of more than 2^45 elements asks for one), while the largest
    dimensions the ABI accepts still plan: 2^31 - 1024 rows in 256 x 256
    tiles, 2^31 - 1024 columns in 128 x 128 general tiles."""
    big = (1 << 31) - 1024
    for bt in (False, True):
        for shape in [(1 << 24, 1 << 24, 1), (big, big, 1)]:
            with pytest.raises(tlg.TlgError) as e:
                tlg.plan(*shape, trans_b=bt)
            assert e.value.status == nat.TLG_ERROR_NOT_SUPPORTED
    assert tlg.plan(1 << 22, 1 << 22, 64)["grid"] == 1 << 30
    p = tlg.plan(big, 8, 8)
    assert p["variant_name"] == "tiled_pipe" and p["grid"] == (big + 255) // 256
    p = tlg.plan(1, big, 1)
    assert p["variant_name"] == "tiled_general" and p["grid"] == (big + 127) // 128
