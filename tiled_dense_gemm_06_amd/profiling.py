"""HBM traffic of a kernel from rocprofv3 counters, for the benchmark's roofline record.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report KiB per
dispatch. Those counters do not read true bytes on every part, so they are
scaled by what the same counters read for a plain device-to-device copy of a
known size (``bench.py --copy-calibration MIB``): factor = copy bytes /
counter bytes, separately for reads and writes.

Usage (after the counter runs, on the CSV files rocprofv3 wrote)::

    python -m tiled_dense_gemm_06_amd.profiling traffic --workload square8192 \\
        --kernel k_tiled_pipe --config pipe_256x256x64_w2x4_s2_a3_early --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-mib 512

It records the scaled fetch and write bytes per launch in
``profiles/traffic.json``, with the tile configuration that ran and the
digest of that kernel's device sources (its own ``.hip`` file and the two
device headers); ``bench.py`` reports them only while the workload still
runs that configuration and those sources still have that digest.

``counters`` writes the Markdown summary of counter passes of one kernel
(the sustained clock, matrix-core occupancy, LDS bank conflicts and the
kernel's resources) for ``profiles/``::

    python -m tiled_dense_gemm_06_amd.profiling counters --workload square8192 \
        --kernel k_tiled_pipe16 --pmc DIR/run_counter_collection.csv --pass-cmd "..." --out FILE

``summary`` writes the Markdown summary of one workload's profile (the
kernel-trace statistics of a command, and the scaled counter bytes when
given) for ``profiles/``::

    python -m tiled_dense_gemm_06_amd.profiling summary --workload square8192 \
        --kernel k_tiled_pipe --trace DIR --trace-cmd "..." [--fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --copy-mib 512 --counter-cmd "..."] --out FILE
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_KERNEL = "copyBuffer"


# the file each kernel's device code lives in (besides the device headers)
KERNEL_FILES = {
    "k_tiled_pipe": "gemm_relu_pipe_gfx950.hip",
    "k_tiled_pipe16": "gemm_relu_pipe16_gfx950.hip",
    "k_tiled_dma": "gemm_relu_gfx950.hip",
    "k_tiled_general": "gemm_relu_gfx950.hip",
    "k_skinny_strip": "gemm_relu_skinny_gfx950.hip",
    "k_streamk": "gemm_relu_streamk_gfx950.hip",
    "k_mx": "gemm_relu_mx_gfx950.hip",
    "k_pingpong": "gemm_relu_pingpong_gfx950.hip",
}
DEVICE_HEADERS = ["gfx950_ops.h", "tile_layout.h"]


def kernel_sources(kernel: str) -> list[str]:
    """The sources a kernel's device code is built from."""
    if kernel not in KERNEL_FILES:
        raise KeyError(f"unknown kernel {kernel!r}; known: {sorted(KERNEL_FILES)}")
    return [os.path.join(HERE, "csrc", f) for f in [KERNEL_FILES[kernel]] + DEVICE_HEADERS]


def kernel_source_digest(kernel: str) -> str:
    """sha256 over the sources a kernel's device code is built from."""
    h = hashlib.sha256()
    for p in kernel_sources(kernel):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_values(path: str, counter: str, kernel_substr: str) -> list[float]:
    """Per-dispatch values of one counter for dispatches whose kernel name contains kernel_substr."""
    out = []
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and kernel_substr in row["Kernel_Name"]:
                out.append(float(row["Counter_Value"]))
    if not out:
        raise ValueError(f"no {counter} rows for a kernel matching {kernel_substr!r} in {path}")
    return out


def mean(xs):
    return sum(xs) / len(xs)


def traffic(args) -> dict:
    copy_bytes = args.copy_mib << 20
    f_copy = counter_values(args.copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    w_copy = counter_values(args.copy_write, "WRITE_SIZE", COPY_KERNEL)
    # the last launches are the timed copies of copy_bytes (earlier ones fill the source)
    fetch_factor = copy_bytes / (f_copy[-1] * 1024.0)
    write_factor = copy_bytes / (w_copy[-1] * 1024.0)
    fetch = mean(counter_values(args.fetch, "FETCH_SIZE", args.kernel)) * 1024.0 * fetch_factor
    write = mean(counter_values(args.write, "WRITE_SIZE", args.kernel)) * 1024.0 * write_factor
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    if "kernel_source_sha256" in data:  # records of the earlier whole-library digest
        data = {}
    data.setdefault("workloads", {})
    data["calibration"] = {"copy_bytes": copy_bytes, "fetch_factor": fetch_factor, "write_factor": write_factor}
    rec = {"kernel": args.kernel, "config": args.config, "sources_sha256": kernel_source_digest(args.kernel),
           "fetch_bytes": fetch, "write_bytes": write, "bytes_per_launch": fetch + write}
    data["workloads"][args.workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def measured_traffic(workload: str, config: str):
    """Scaled HBM bytes per launch for a workload, if they were taken with the
    tile configuration ``config`` on the kernel's current sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get("workloads", {}).get(workload)
    if not rec or rec.get("config") != config or rec.get("kernel") not in KERNEL_FILES:
        return None
    if rec.get("sources_sha256") != kernel_source_digest(rec["kernel"]):
        return None
    return rec.get("bytes_per_launch")


PEAK_MFMA_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PEAK_MX_TFLOPS = {"e4m3": 5000.0, "e5m2": 5000.0, "e2m1": 10100.0}  # dense block-scaled MFMA


def _stats_rows(trace_dir: str):
    with open(os.path.join(trace_dir, "run_kernel_stats.csv")) as f:
        return list(csv.DictReader(f))


def _median_ns(trace_dir: str) -> dict:
    """Median dispatch duration (ns) per kernel name, from the per-dispatch
    trace (run_kernel_trace.csv), if the trace directory holds one."""
    path = os.path.join(trace_dir, "run_kernel_trace.csv")
    if not os.path.exists(path):
        return {}
    durs = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            durs.setdefault(row["Kernel_Name"], []).append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    out = {}
    for name, d in durs.items():
        d.sort()
        n = len(d)
        out[name] = d[n // 2] if n % 2 else 0.5 * (d[n // 2 - 1] + d[n // 2])
    return out


def summary(args) -> str:
    from . import workloads as wl

    w = wl.WORKLOADS[args.workload]
    # block-scaled (--mx): codes of 1 or 1/2 byte, one scale byte per 32 k, fp16 C
    if args.mx:
        bits = 4 if args.mx == "e2m1" else 8
        alg_bytes = (w.M + w.N) * w.K * bits // 8 + (w.M + w.N) * (w.K // 32) + 2 * w.M * w.N
        peak, peak_name = PEAK_MX_TFLOPS[args.mx], f"{args.mx} block-scaled dense"
        what = f"{args.mx} codes of A and B, their scale bytes and fp16 C once"
    else:
        alg_bytes, peak, peak_name, what = w.alg_bytes, PEAK_MFMA_TFLOPS, "fp16 dense", "A, B and C once"
    rows = _stats_rows(args.trace)
    med = _median_ns(args.trace)
    main = [r for r in rows if args.kernel in r["Name"]]
    if not main:
        raise ValueError(f"no kernel matching {args.kernel!r} in {args.trace}")
    r0 = max(main, key=lambda r: int(r["Calls"]))
    avg_ns = float(r0["AverageNs"])
    lines = [f"# {args.title or args.kernel} — workload {w.name}", ""]
    lines += ["Kernel trace (from the repository root, on one MI355X):", "", "    " + args.trace_cmd, ""]
    lines += ["| kernel | calls | avg ns | median ns | min ns | max ns |", "|---|---|---|---|---|---|"]
    for r in rows:
        m = med.get(r["Name"])
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):,.0f} | "
                     f"{'' if m is None else f'{m:,.0f}'} | {float(r['MinNs']):,.0f} | {float(r['MaxNs']):,.0f} |")
    lines.append("")
    if args.note:
        lines += [args.note, ""]
    tflops = w.flop / (avg_ns * 1e-9) / 1e12
    gbs = alg_bytes / (avg_ns * 1e-9) / 1e9
    lines.append(f"From the trace average ({avg_ns / 1e3:,.1f} us per launch): {tflops:,.1f} TFLOP/s "
                 f"({100 * tflops / peak:.1f} % of the {peak} TFLOP/s {peak_name} peak), "
                 f"{gbs:,.0f} GB/s of algorithmic bytes ({alg_bytes:,} B: {what}; "
                 f"{100 * gbs / PEAK_HBM_GBS:.1f} % of {PEAK_HBM_GBS:.0f} GB/s).")
    m0 = med.get(r0["Name"])
    if m0:
        lines.append("")
        lines.append(f"From the trace median ({m0 / 1e3:,.1f} us per launch): "
                     f"{w.flop / (m0 * 1e-9) / 1e12:,.1f} TFLOP/s ({100 * w.flop / (m0 * 1e-9) / 1e12 / peak:.1f} %), "
                     f"{alg_bytes / (m0 * 1e-9) / 1e9:,.0f} GB/s "
                     f"({100 * alg_bytes / (m0 * 1e-9) / 1e9 / PEAK_HBM_GBS:.1f} % of {PEAK_HBM_GBS:.0f} GB/s).")
    lines.append("")
    if args.fetch:
        copy_bytes = args.copy_mib << 20
        ff = copy_bytes / (counter_values(args.copy_fetch, "FETCH_SIZE", COPY_KERNEL)[-1] * 1024.0)
        wf = copy_bytes / (counter_values(args.copy_write, "WRITE_SIZE", COPY_KERNEL)[-1] * 1024.0)
        fetch = mean(counter_values(args.fetch, "FETCH_SIZE", args.kernel)) * 1024.0 * ff
        write = mean(counter_values(args.write, "WRITE_SIZE", args.kernel)) * 1024.0 * wf
        lines += ["HBM counters, one pass each (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch):", "",
                  "    " + args.counter_cmd.replace("COUNTERDIR", "fetch").replace("COUNTER", "FETCH_SIZE"),
                  "    " + args.counter_cmd.replace("COUNTERDIR", "write").replace("COUNTER", "WRITE_SIZE"), "",
                  f"scaled by a plain {args.copy_mib} MiB device copy measured the same way "
                  f"(`python3 bench.py --copy-calibration {args.copy_mib} --steps 3 --warmup 1` under each "
                  f"counter): fetch factor {ff:.4f}, write factor {wf:.4f}.", "",
                  "| per launch | bytes | x algorithmic |", "|---|---|---|",
                  f"| fetched from beyond L2 | {fetch:,.0f} | {fetch / alg_bytes:.2f} |",
                  f"| written | {write:,.0f} | {write / alg_bytes:.2f} |",
                  f"| total (`traffic`) | {fetch + write:,.0f} | {(fetch + write) / alg_bytes:.2f} |", ""]
    text = "\n".join(lines)
    with open(args.out, "w") as f:
        f.write(text)
    return text


def _dispatches(path: str, kernel_substr: str) -> list[dict]:
    """Per-dispatch counter values, duration (ns) and resources of the
    dispatches of one kernel in a rocprofv3 --pmc CSV file."""
    per = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if kernel_substr not in row["Kernel_Name"]:
                continue
            d = per.setdefault(row["Dispatch_Id"], {
                "name": row["Kernel_Name"], "ns": int(row["End_Timestamp"]) - int(row["Start_Timestamp"]),
                "vgpr": int(row["VGPR_Count"]), "agpr": int(row["Accum_VGPR_Count"]),
                "sgpr": int(row["SGPR_Count"]), "lds": int(row["LDS_Block_Size"]),
                "scratch": int(row["Scratch_Size"]), "wg": int(row["Workgroup_Size"]),
                "grid": int(row["Grid_Size"]), "counters": {}})
            d["counters"][row["Counter_Name"]] = float(row["Counter_Value"])
    if not per:
        raise ValueError(f"no dispatch of a kernel matching {kernel_substr!r} in {path}")
    return list(per.values())


def counters(args) -> str:
    """Markdown summary of counter passes of one kernel on one workload: mean
    per dispatch of every counter, and what follows from them: the sustained
    shader clock (GRBM_GUI_ACTIVE summed over the 8 XCDs, per dispatch
    duration), the matrix-core occupancy (SQ_VALU_MFMA_BUSY_CYCLES summed over
    the 1024 SIMDs, per SIMD-cycle of the dispatch), LDS bank-conflict cycles
    per LDS instruction; and the kernel's resources from the same records."""
    from . import workloads as wl

    w = wl.WORKLOADS[args.workload]
    lines = [f"# {args.title or args.kernel} — counters, workload {w.name}", "",
             "Counter passes (from the repository root, on one MI355X; one rocprofv3 run per pass):", ""]
    lines += ["    " + c for c in args.pass_cmds]
    lines += [""]
    merged = {}
    res = None
    for path in args.pmc:
        ds = _dispatches(path, args.kernel)
        res = res or ds[0]
        for k in ds[0]["counters"]:
            merged[k] = (mean([d["counters"][k] for d in ds]), mean([d["ns"] for d in ds]), len(ds))
    lines += [f"Kernel: `{res['name']}`", "",
              f"Resources per work-group of {res['wg']} threads ({res['grid'] // max(1, res['wg'])} work-groups): "
              f"{res['vgpr']} VGPRs and {res['agpr']} AGPRs per lane (as the trace reports them), {res['sgpr']} SGPRs, "
              f"{res['lds']:,} bytes of LDS, {res['scratch']} bytes of scratch per lane.", "",
              "| counter | mean per dispatch | dispatches | mean dispatch ns |", "|---|---|---|---|"]
    for k in sorted(merged):
        v, ns, n = merged[k]
        lines.append(f"| {k} | {v:,.0f} | {n} | {ns:,.0f} |")
    lines.append("")
    derived = []
    if "GRBM_GUI_ACTIVE" in merged:
        gui, ns, _ = merged["GRBM_GUI_ACTIVE"]
        ghz = gui / 8 / ns
        derived.append(f"sustained shader clock: {ghz:.3f} GHz (GRBM_GUI_ACTIVE / 8 XCDs / dispatch ns)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in merged:
            busy = merged["SQ_VALU_MFMA_BUSY_CYCLES"][0] / 1024 / (gui / 8)
            derived.append(f"matrix cores busy: {100 * busy:.1f} % of the SIMD-cycles of the dispatch "
                           f"(SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / GPU-busy cycles per XCD); at the sustained "
                           f"clock that is {busy * ghz / 2.4 * 100:.1f} % of the 2.4 GHz dense peak")
    if "SQ_LDS_BANK_CONFLICT" in merged and "SQ_INSTS_LDS" in merged and merged["SQ_INSTS_LDS"][0] > 0:
        derived.append(f"LDS bank-conflict cycles per LDS instruction: "
                       f"{merged['SQ_LDS_BANK_CONFLICT'][0] / merged['SQ_INSTS_LDS'][0]:.3f}")
    if derived:
        lines += ["Derived:", ""] + [f"* {x}" for x in derived] + [""]
    if args.note:
        lines += [args.note, ""]
    text = "\n".join(lines)
    with open(args.out, "w") as f:
        f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_FILES), help="the kernel (name prefix)")
    t.add_argument("--config", required=True, help="the tile configuration that ran (tlg.plan's config_name)")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    m = sub.add_parser("summary")
    m.add_argument("--workload", required=True)
    m.add_argument("--kernel", required=True, help="substring of the kernel name")
    m.add_argument("--title", default="")
    m.add_argument("--trace", required=True, help="rocprofv3 --kernel-trace --stats output directory")
    m.add_argument("--trace-cmd", required=True)
    m.add_argument("--note", default="")
    m.add_argument("--fetch")
    m.add_argument("--write")
    m.add_argument("--copy-fetch")
    m.add_argument("--copy-write")
    m.add_argument("--copy-mib", type=int, default=512)
    m.add_argument("--counter-cmd", default="")
    m.add_argument("--mx", choices=sorted(PEAK_MX_TFLOPS), help="the block-scaled path with these codes")
    m.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--workload", required=True)
    c.add_argument("--kernel", required=True, help="substring of the kernel name")
    c.add_argument("--title", default="")
    c.add_argument("--pmc", action="append", required=True, help="a rocprofv3 --pmc counter_collection CSV")
    c.add_argument("--pass-cmd", action="append", default=[], dest="pass_cmds",
                   help="the command of each counter pass")
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    args = ap.parse_args()
    if args.cmd == "traffic":
        print(json.dumps(traffic(args)))
    elif args.cmd == "counters":
        counters(args)
    else:
        summary(args)


if __name__ == "__main__":
    main()
