"""MFMA result hazards in the generated assembly (CPU only: hipcc -S).

The 16 x 16 x 32 kernel writes its MFMAs as inline assembly, so the compiler
adds no wait states behind them; these tests compile every kernel source for
gfx950 with the library's own flags and check, with ``tests/mfma_hazards.py``,
that no instruction the compiler placed (a copy or spill of an accumulator)
touches an MFMA's result before the matrix core has written it, and that no
load (the inline-assembly direct-to-LDS ones included) reads a scalar
register, such as a buffer descriptor reloaded from a spill, too soon after a
vector-ALU instruction wrote it. The scanners themselves are checked first on
small listings with planted hazards.
"""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import mfma_hazards as mh  # noqa: E402

from tiled_dense_gemm_06_amd import build as B  # noqa: E402

MFMA = "v_mfma_f32_16x16x32_f16 a[4:7], v[0:3], v[8:11], a[4:7]"


def test_scanner_flags_a_copy_right_behind_the_mfma():
    assert mh.scan([MFMA, "v_accvgpr_read_b32 v20, a5", "s_endpgm"]) == \
        [(0, "v_accvgpr_read_b32 v20, a5", "a5")]
    # a write of the destination (a spill slot reused) is flagged too
    assert len(mh.scan([MFMA, "v_accvgpr_write_b32 a6, v1", "s_endpgm"])) == 1


def test_scanner_counts_wait_states():
    nops = ["s_nop 7", "s_nop 7", "s_nop 7"]
    assert mh.scan([MFMA, *nops, "v_accvgpr_read_b32 v20, a5", "s_endpgm"]) == []
    # 17 wait states are one short of the 18 the MFMA needs
    assert len(mh.scan([MFMA, "s_nop 7", "s_nop 7", "v_mov_b32 v1, 0", "v_accvgpr_read_b32 v20, a5"])) == 1
    assert mh.scan([MFMA, "s_nop 7", "s_nop 7", "v_mov_b32 v1, 0", "v_mov_b32 v2, 0",
                    "v_accvgpr_read_b32 v20, a5"]) == []
    # other registers are free at once
    assert mh.scan([MFMA, "v_accvgpr_read_b32 v20, a8", "s_endpgm"]) == []


def test_scanner_accepts_accumulation_in_place_but_not_other_reads():
    assert mh.scan([MFMA, MFMA, "s_endpgm"]) == []
    other = "v_mfma_f32_16x16x32_f16 a[8:11], v[4:7], v[8:11], a[4:7]"  # reads a[4:7] as its accumulator input
    assert len(mh.scan([MFMA, other, "s_endpgm"])) == 4


def test_scanner_follows_branches():
    # debt carried along a taken branch and along a fall-through
    lines = [MFMA, "s_cbranch_scc1 .LBB0_2", "s_nop 7", "s_nop 7", "s_nop 7", ".LBB0_2:",
             "v_accvgpr_read_b32 v20, a4", "s_endpgm"]
    assert len(mh.scan(lines)) == 1
    lines = [MFMA, "s_branch .LBB0_2", ".LBB0_1:", "v_accvgpr_read_b32 v20, a4", "s_endpgm", ".LBB0_2:",
             "s_nop 7", "s_nop 7", "s_nop 7", "s_branch .LBB0_1"]
    assert mh.scan(lines) == []
    lines = [MFMA, "s_branch .LBB0_1", ".LBB0_1:", "v_accvgpr_read_b32 v20, a4", "s_endpgm"]
    assert len(mh.scan(lines)) == 1


def test_sgpr_scanner_flags_a_reload_right_before_a_load():
    reload = "v_readlane_b32 s1, v255, 25"
    load = "buffer_load_dwordx4 v0, s[0:3], 0 offen lds"
    assert mh.scan_sgpr_vmem([reload, "s_nop 0", load, "s_endpgm"]) == [(0, load, "s1")]
    # five wait states are enough; a scalar write of the register is not a hazard
    assert mh.scan_sgpr_vmem([reload, "s_nop 4", load, "s_endpgm"]) == []
    assert mh.scan_sgpr_vmem(["s_mov_b32 s1, 0", load, "s_endpgm"]) == []
    # carried along a branch
    assert len(mh.scan_sgpr_vmem([reload, "s_branch .LBB0_1", ".LBB0_1:", load, "s_endpgm"])) == 1


def _compile_asm(src, out_path):
    flags = [f for f in B.HIP_FLAGS if f != "-shared"]
    cmd = [B.hipcc(), *flags, *B.SOURCE_FLAGS.get(os.path.basename(src), []), "-I", B.INCLUDE, "-I", B.CSRC, "-S",
           "--offload-device-only", src, "-o", out_path]
    return subprocess.run(cmd, capture_output=True, text=True)


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    """The assembly of every kernel source, compiled with the library's flags:
    {source file name: {function: lines}}."""
    srcs = [s for s in B.SOURCES if s.endswith(".hip")]
    d = tmp_path_factory.mktemp("asm")
    outs = [str(d / (os.path.basename(s) + ".s")) for s in srcs]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = list(ex.map(_compile_asm, srcs, outs))
    for src, r in zip(srcs, results):
        assert r.returncode == 0, f"hipcc -S {os.path.basename(src)}:\n{r.stderr[-2000:]}"
    return {os.path.basename(src): mh.functions(open(out).read()) for src, out in zip(srcs, outs)}


def test_inline_asm_mfma_results_are_never_read_early(listings):
    srcs = [n for n in listings if re.search(r'asm\s+volatile\s*\(\s*"v_mfma', open(os.path.join(B.CSRC, n)).read())]
    assert srcs, "the 16 x 16 x 32 kernel writes its MFMAs as inline assembly"
    found = []
    kernels = 0
    for n in srcs:
        for name, lines in listings[n].items():
            if not any(ln.startswith("v_mfma") for ln in lines):
                continue
            kernels += 1
            found += [(name, ins, reg) for _, ins, reg in mh.scan(lines)]
    assert kernels >= 10
    assert not found, f"{len(found)} early uses of MFMA results, e.g. {found[:4]}"


def test_loads_never_read_a_fresh_vector_written_scalar(listings):
    """No vector memory instruction in any kernel reads a scalar register
    (a buffer descriptor, a scalar offset) within five wait states of a
    vector-ALU write of it, the inline-assembly direct-to-LDS loads included."""
    found = []
    for n, fns in listings.items():
        for name, lines in fns.items():
            found += [(n, name, ins, reg) for _, ins, reg in mh.scan_sgpr_vmem(lines)]
    assert not found, f"{len(found)} loads too close to a scalar register's vector write, e.g. {found[:4]}"
