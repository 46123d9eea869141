"""profiles/ summaries from rocprofv3 CSV output (tiled_dense_gemm_06_amd.profiling),
on synthetic trace and counter files, without a GPU: the per-kernel median
from the per-dispatch trace, the rates at the trace average and median, and
the copy-calibrated HBM bytes."""
import argparse
import csv
import os

from tiled_dense_gemm_06_amd import profiling as pr
from tiled_dense_gemm_06_amd import workloads as wl

KERNEL = "void tlg::k_tiled_dma<tlg::TileShape<64, 64, 64, 2, 2, 3>, false, false>(tlg::KArgs)"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_summary_reports_median_and_scaled_traffic(tmp_path):
    trace = tmp_path / "trace"
    trace.mkdir()
    durs = [4000, 4100, 3900, 9000, 4050]  # ns; one slow launch
    _write(trace / "run_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                            "MaxNs", "StdDev"],
           [[KERNEL, len(durs), sum(durs), sum(durs) / len(durs), 100.0, min(durs), max(durs), 0.0]])
    _write(trace / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[KERNEL, 1000 * i, 1000 * i + d] for i, d in enumerate(durs)])
    assert pr._median_ns(str(trace)) == {KERNEL: 4050}
    # counters: the kernel fetched 3 MiB and wrote 1 MiB per dispatch (as read);
    # the 512 MiB copy read 256 MiB and wrote 512 MiB worth of counter KiB
    cnt_header = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(tmp_path / "f.csv", cnt_header, [[KERNEL, "FETCH_SIZE", 3072.0]] * 2)
    _write(tmp_path / "w.csv", cnt_header, [[KERNEL, "WRITE_SIZE", 1024.0]] * 2)
    _write(tmp_path / "cf.csv", cnt_header, [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 256.0 * 1024]])
    _write(tmp_path / "cw.csv", cnt_header, [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 512.0 * 1024]])
    out = tmp_path / "summary.md"
    args = argparse.Namespace(workload="square256", kernel="k_tiled_dma", title="dma_64x64x64_w2x2_s3 (k_tiled_dma)",
                              trace=str(trace), trace_cmd="rocprofv3 ...", note="", fetch=str(tmp_path / "f.csv"),
                              write=str(tmp_path / "w.csv"), copy_fetch=str(tmp_path / "cf.csv"),
                              copy_write=str(tmp_path / "cw.csv"), copy_mib=512, counter_cmd="rocprofv3 --pmc COUNTER",
                              mx=None, out=str(out))
    text = pr.summary(args)
    assert os.path.exists(out)
    w = wl.WORKLOADS["square256"]
    avg = sum(durs) / len(durs)
    assert f"From the trace average ({avg / 1e3:,.1f} us per launch)" in text
    assert "From the trace median (4.0 us per launch)" in text or "From the trace median (4.1 us per launch)" in text
    assert f"{w.flop / (4050e-9) / 1e12:,.1f} TFLOP/s" in text
    # fetch factor 2 (copy read 512 MiB, counter 256 MiB), write factor 1
    assert f"| fetched from beyond L2 | {3 * 2 ** 20 * 2:,} |" in text
    assert f"| written | {2 ** 20:,} |" in text


def test_counters_derives_clock_occupancy_and_conflicts(tmp_path):
    # two dispatches of one kernel, 1 ms each, at 1.5 GHz on 8 XCDs with the
    # 1024 SIMDs' matrix cores busy 60 % of the cycles; one copy dispatch that
    # the kernel filter must skip
    header = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
              "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
              "End_Timestamp"]
    cycles = 1.5e6 * 8  # GRBM_GUI_ACTIVE over 8 XCDs for 1 ms at 1.5 GHz
    rows = []
    for d in (1, 2):
        res = [d, KERNEL, 1024 * 256, 256, 65536, 0, 128, 256, 96]
        t0 = 10_000_000 * d
        for name, v in (("GRBM_GUI_ACTIVE", cycles), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.6 * 1024 * cycles / 8),
                        ("SQ_INSTS_LDS", 1000.0), ("SQ_LDS_BANK_CONFLICT", 250.0)):
            rows.append(res + [name, v, t0, t0 + 1_000_000])
    rows.append([3, "__amd_rocclr_copyBuffer", 512, 512, 0, 0, 8, 0, 32, "GRBM_GUI_ACTIVE", 5.0, 0, 10])
    _write(tmp_path / "sq.csv", header, rows)
    out = tmp_path / "counters.md"
    args = argparse.Namespace(workload="square256", kernel="k_tiled_dma", title="", pmc=[str(tmp_path / "sq.csv")],
                              pass_cmds=["rocprofv3 --pmc ..."], note="a note", out=str(out))
    text = pr.counters(args)
    assert os.path.exists(out)
    assert "1024 work-groups" in text and "128 VGPRs and 256 AGPRs" in text and "65,536 bytes of LDS" in text
    assert "| GRBM_GUI_ACTIVE | 12,000,000 | 2 | 1,000,000 |" in text
    assert "sustained shader clock: 1.500 GHz" in text
    assert "matrix cores busy: 60.0 %" in text and "37.5 % of the 2.4 GHz dense peak" in text
    assert "bank-conflict cycles per LDS instruction: 0.250" in text
    assert text.rstrip().endswith("a note")


def test_committed_traffic_matches_the_current_kernels():
    """Every workload's HBM traffic record in profiles/traffic.json was taken
    on the tile configuration the planner picks today and on the kernel
    sources as they stand (a source change voids the record, and the
    benchmark line then reports no traffic)."""
    import tiled_dense_gemm_06_amd as tlg
    from tiled_dense_gemm_06_amd import workloads as wl
    from tiled_dense_gemm_06_amd.profiling import measured_traffic
    for name in ("square256", "square4096", "ragged3001x2049x1537", "skinny16x14336x4096", "square8192"):
        w = wl.WORKLOADS[name]
        cfg = tlg.plan(w.M, w.N, w.K)["config_name"]
        t = measured_traffic(name, cfg)
        assert t is not None and t > 0, (name, cfg)
