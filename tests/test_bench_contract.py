"""bench.py's output contract: one JSON line with the fields the benchmark
record needs (metric, value, roofline, cpu_baseline, ...), the refusal of
more than one GPU, and the host-side pieces (the oracle's timed sample, the
device's sysfs record) that run without a GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tiled_dense_gemm_06_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_cpu_baseline_record():
    """The oracle timed on whole sampled rows: the record's fields, a sample
    of whole thread batches, and the single-thread time of the 256^3 problem."""
    w = wl.WORKLOADS["square256"]
    A, B = wl.make_inputs(w)
    rec = bench.cpu_baseline(w, A, B, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOPS"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "output rows" in rec["sample"] and f"on {rec['cores']} threads" in rec["sample"]
    st = rec["single_thread_square256"]
    assert st["seconds"] > 0 and st["value"] == pytest.approx(2 * 256 ** 3 / st["seconds"] / 1e12)


def test_sysfs_info_without_a_node():
    class NoPci:
        pass

    class Missing:
        pci_domain_id, pci_bus_id, pci_device_id = 0xFFFF, 0xFF, 0x1F

    for props in (NoPci(), Missing()):
        assert bench.gpu_sysfs_info(props) == {"sclk_peak_mhz": None, "compute_partition": None,
                                               "memory_partition": None}


CONTRACT = {"metric": str, "value": float, "unit": str, "n_gpus": int, "steps": int, "warmup": int,
            "ms_per_step": float, "higher_is_better": bool, "scaling": str, "dtype": str, "data": str,
            "config": dict, "roofline": dict}


@pytest.mark.gpu
@pytest.mark.parametrize("extra", [[], ["--eager"]])
def test_bench_json_line(extra):
    """One short bench run of the 4096^3 workload (graph-timed and eager): a
    single JSON line with every contract field, a roofline record whose rate
    is the algorithmic FLOP over the timed launch, and the oracle baseline."""
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "square4096", "--steps", "5",
           "--warmup", "2", "--cpu-seconds", "0.5", *extra]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    out = json.loads(lines[0])
    for key, typ in CONTRACT.items():
        assert isinstance(out[key], typ), key
    assert out["n_gpus"] == 1 and out["steps"] == 5 and out["warmup"] == 2
    assert out["higher_is_better"] is True and out["scaling"] == "weak" and out["vs_baseline"] is None
    assert out["config"]["workload"] == "square4096"
    assert out["config"]["timing"] == ("events_per_launch" if extra else "hip_graph")
    w = wl.WORKLOADS["square4096"]
    assert out["value"] == pytest.approx(w.flop / (out["ms_per_step"] * 1e-3) / 1e12, rel=1e-6)
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == pytest.approx(2516.5824)
    assert roof["achieved"] == pytest.approx(w.flop / (roof["launch_ms_avg"] * 1e-3) / 1e12, rel=1e-6)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    assert roof["traffic"] is None or roof["traffic"] > w.alg_bytes
    cb = out["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOPS" and cb["cores"] >= 1 and cb["value"] > 0
    if extra:
        assert "skinny" not in out and "vendor_reference" not in out
    else:
        sk = out["skinny"]  # the HBM-bound workload, after the timed steps
        s4 = wl.WORKLOADS["skinny16x14336x4096"]
        assert sk["workload"] == s4.name and sk["unit"] == "GB/s" and sk["peak"] == 8000.0
        assert sk["achieved"] == pytest.approx(s4.alg_bytes / (sk["us_per_call"] * 1e-6) / 1e9, rel=1e-6)
        assert sk["frac"] == pytest.approx(sk["achieved"] / 8000.0)
        assert sk["timing"] == "hip_graph" and sk["rotated_buffers"] >= 5


@pytest.mark.gpu
def test_bench_vendor_reference_at_8192():
    """The default 8192^3 run adds the interleaved vendor-BLAS reference:
    per-call times of both sides over the same rounds."""
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--no-cpu-baseline"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    out = json.loads([ln for ln in r.stdout.splitlines() if ln.strip()][-1])
    vr = out["vendor_reference"]
    assert vr["rounds"] >= 2 and vr["calls_per_round"] >= 10
    for side in ("tlg", "vendor_matmul"):
        assert 0 < vr[side]["best"] <= vr[side]["median"]
    assert vr["tlg_vs_vendor_matmul_best"] == pytest.approx(vr["vendor_matmul"]["best"] / vr["tlg"]["best"])
    assert "skinny" in out and "cpu_baseline" not in out
