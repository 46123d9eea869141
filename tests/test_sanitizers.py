"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (no GPU).

* The CPU oracles (oracle/oracle.c, oracle/oracle_mx.c) are built with gcc
  and the sanitizers together with tests/sanitize/oracle_driver.c, which
  calls every oracle function on random small problems and checks that the
  oracle's forms agree.
* The library is built with hipcc with the sanitizers on its host code only
  (each sanitizer flag placed after -Xarch_host; the GPU code is compiled as
  usual and never runs here), and tests/sanitize/plan_driver.cpp drives its
  planners and argument checks over edge and random arguments.

Any invalid memory access, leak, signed overflow, invalid enum load or
other undefined behaviour aborts the driver (-fno-sanitize-recover=all), so
the test fails with the sanitizer's report.
"""
import os
import shutil
import subprocess

import pytest

from tiled_dense_gemm_06_amd import build as tlg_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-pthread", *SAN_FLAGS,
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(ROOT, "oracle", "oracle_mx.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"), timeout=600)
    assert "oracle_driver: ok" in r.stdout


@pytest.mark.skipif(shutil.which(tlg_build.hipcc()) is None and not os.path.exists(tlg_build.hipcc()),
                    reason="hipcc not found")
def test_planner_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libtlg_san.so")
    host_san = []
    for f in SAN_FLAGS:
        host_san += ["-Xarch_host", f]
    # the GPU code keeps the library's own flags (its inline assembly needs
    # the optimised register allocation); the host code is built for debugging
    _run(tlg_build.compile_cmd(lib, ["-Xarch_host", "-O1", "-Xarch_host", "-g", *host_san]), timeout=1200)
    exe = str(tmp_path / "plan_driver")
    _run([tlg_build.hipcc(), "-O1", "-g", "-std=c++17", *host_san, "-I", tlg_build.INCLUDE,
          os.path.join(SAN, "plan_driver.cpp"), "-L", str(tmp_path), "-ltlg_san",
          "-Wl,-rpath," + str(tmp_path), "-o", exe], timeout=600)
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"), timeout=600)
    assert "plan_driver: ok" in r.stdout
