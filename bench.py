#!/usr/bin/env python3
"""Throughput of C = ReLU(A.B) (fp16 in, fp32 accumulation, fp16 out) on one
MI355X, through the tlg C ABI.

One step is one full call of the path on one batch of synthetic input that is
already resident in HBM. The default workload is M = N = K = 8192 with
U[-1,1] inputs from seed 4. The other workloads are accepted with
--workload for measurement runs; the parity tests cover them all.

The timed steps are captured in a HIP graph and one replay is timed between
two HIP events on the launch stream (--eager: each step launched from the
host between its own pair of events instead).

Prints one JSON line: the contract fields, plus
  roofline     - the dominant kernel's achieved rate (algorithmic FLOP or bytes
                 per launch / its average launch duration from HIP events on
                 the stream it runs on: the replay time over the steps, or the
                 mean of the per-launch event pairs with --eager) against the
                 MI355X peak;
  skinny       - (default run) the HBM-bound workload M = 16, N = 14336,
                 K = 4096 timed the same way after the main steps: us per
                 call, algorithmic GB/s and the fraction of 8 TB/s;
  vendor_reference - (default run at 8192^3) this library's call and the
                 vendor BLAS's plain fp16 matmul interleaved on the same
                 inputs, after the timed steps;
  cpu_baseline - the CPU oracle timed on a bounded sample of the same workload
                 (sampled output rows), in the same unit.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM+ReLU TFLOPS (fp16 in, fp32 acc) at 8192³ and % of fp16 MFMA peak"
# MI355X dense fp16 MFMA: 256 CUs x 4096 FLOP/clock/CU x 2.4 GHz = 2516.6 TFLOP/s (AMD's "2.5 PF")
PEAK_MFMA_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20  # MI355X Infinity Cache; rotated buffers exceed twice this
def time_steps(torch, step, steps: int, warmup: int, graph: bool) -> dict:
    """Run `warmup` untimed steps, then time `steps` steps on the current stream.

    step(i, stream) enqueues step i on `stream`. With graph=True the timed
    steps are captured once into a HIP graph and replayed (one untimed
    replay, then one timed replay between two events on the launch stream),
    so the device runs them back to back without the host's per-call launch
    cost; every launch's average duration is then the replay time / steps.
    With graph=False each step is bracketed by its own pair of events."""
    import numpy as np

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i, stream)
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for i in range(steps):
                step(i, cs)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / steps
        del g
        return {"ms_per_step": ms, "launch_ms_avg": ms, "launch_ms_min": None, "wall": wall, "timing": "hip_graph"}
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step(i, stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return {"ms_per_step": starts[0].elapsed_time(ends[-1]) / steps,
            "launch_ms_avg": float(np.mean(per_launch_ms)), "launch_ms_min": float(np.min(per_launch_ms)),
            "wall": wall, "timing": "events_per_launch"}


def rotated_inputs(torch, w, dev, A, B):
    """R copies of the workload's A, B and C, R chosen so that the working set
    is more than twice the Infinity Cache: every step reads from HBM."""
    R = max(2, math.ceil(2 * MALL_BYTES / w.alg_bytes) + 1)
    Ad0 = torch.from_numpy(A).to(dev)
    Bd0 = torch.from_numpy(B).to(dev)
    As = [Ad0] + [Ad0.clone() for _ in range(R - 1)]
    Bs = [Bd0] + [Bd0.clone() for _ in range(R - 1)]
    Cs = [torch.empty((w.M, w.N), dtype=torch.float16, device=dev) for _ in range(R)]
    return R, As, Bs, Cs


def skinny_record(torch, tlg, wl, dev, steps: int, warmup: int) -> dict:
    """The HBM-bound workload (M = 16, N = 14336, K = 4096) in the default
    plan, graph-timed on rotated inputs: microseconds per call, algorithmic
    bytes per second and the fraction of the 8 TB/s HBM peak."""
    w = wl.WORKLOADS["skinny16x14336x4096"]
    A, B = wl.make_inputs(w)
    R, As, Bs, Cs = rotated_inputs(torch, w, dev, A, B)
    h = tlg.handle_for(dev)

    def step(i, stream):
        tlg.gemm_relu(As[i % R], Bs[i % R], out=Cs[i % R], handle=h, stream=stream)

    tm = time_steps(torch, step, steps, warmup, graph=True)
    us = tm["launch_ms_avg"] * 1e3
    gbs = w.alg_bytes / (us * 1e-6) / 1e9
    plan = tlg.plan(w.M, w.N, w.K)
    return {"workload": w.name, "us_per_call": us, "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "alg_bytes": w.alg_bytes, "steps": steps, "timing": tm["timing"],
            "rotated_buffers": R, "kernel": plan["config_name"], "strip_columns": plan["block_n"],
            "work_groups": plan["grid"]}


def vendor_reference(torch, tlg, w, As, Bs, Cs, R: int, rounds: int, calls: int) -> dict:
    """Outside the timed region: this library's default call and the vendor
    BLAS (torch.matmul, which dispatches to hipBLASLt on this GPU; fp16 in,
    fp16 out, no ReLU, so it does less than this path) on the same rotated
    inputs, interleaved round by round (the order alternates) so that both
    see the same clock and thermal state. Each round times `calls`
    back-to-back calls of one side between two events; reported per call.
    Also the vendor's fused bias + ReLU form (torch._addmm_activation with a
    zero bias) when this torch build provides it."""
    import numpy as np

    dev = As[0].device
    h = tlg.handle_for(dev)
    stream = torch.cuda.current_stream(dev)
    Vs = [torch.empty_like(c) for c in Cs[:R]]
    bias = torch.zeros((w.N,), dtype=torch.float16, device=dev)

    def ours(i):
        tlg.gemm_relu(As[i % R], Bs[i % R], out=Cs[i % R], handle=h, stream=stream)

    def vendor(i):
        torch.matmul(As[i % R], Bs[i % R], out=Vs[i % R])

    def vendor_relu(i):
        Vs[i % R] = torch._addmm_activation(bias, As[i % R], Bs[i % R], use_gelu=False)

    sides = {"tlg": ours, "vendor_matmul": vendor}
    try:
        vendor_relu(0)
        torch.cuda.synchronize()
        sides["vendor_addmm_relu"] = vendor_relu
    except Exception:  # noqa: BLE001 - optional torch entry point
        pass
    for f in sides.values():  # warm-up (and the vendor's heuristics)
        for i in range(3):
            f(i)
    torch.cuda.synchronize()
    times = {k: [] for k in sides}
    names = list(sides)
    for r in range(rounds):
        order = names if r % 2 == 0 else names[::-1]
        for k in order:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(calls):
                sides[k](i)
            e1.record(stream)
            torch.cuda.synchronize()
            times[k].append(e0.elapsed_time(e1) / calls * 1e3)
    out = {"rounds": rounds, "calls_per_round": calls, "unit": "us_per_call",
           "backend": "torch.matmul (hipBLASLt), fp16 out, no ReLU"}
    for k, v in times.items():
        out[k] = {"best": float(np.min(v)), "median": float(np.median(v)),
                  "tflops_best": w.flop / (np.min(v) * 1e-6) / 1e12}
    out["tlg_vs_vendor_matmul_best"] = out["vendor_matmul"]["best"] / out["tlg"]["best"]
    return out


def gpu_sysfs_info(props) -> dict:
    """Peak shader clock (the top level of pp_dpm_sclk, MHz) and the compute and
    memory partition modes of the device, read from its PCI sysfs node; None
    for whatever the node does not show."""
    out = {"sclk_peak_mhz": None, "compute_partition": None, "memory_partition": None}
    try:
        node = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
    except AttributeError:
        return out

    def read(name):
        try:
            with open(os.path.join(node, name)) as f:
                return f.read()
        except OSError:
            return None

    levels = read("pp_dpm_sclk")
    if levels:
        mhz = [int(tok[:-3]) for tok in levels.split() if tok.lower().endswith("mhz") and tok[:-3].isdigit()]
        out["sclk_peak_mhz"] = max(mhz) if mhz else None
    for key, name in (("compute_partition", "current_compute_partition"),
                      ("memory_partition", "current_memory_partition")):
        v = read(name)
        out[key] = v.strip() if v else None
    return out


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "" where unavailable."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(w, A, B, target_s: float):
    """The oracle as it stands, on whole sampled output rows of the workload.

    The oracle splits rows across its threads, so the sample is whole batches
    of one row per thread, grown until one call takes at least half of
    target_s seconds of wall time (the last call is the one reported)."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    n = min(threads, w.M)
    while True:  # grow the sample (4x a round) until it takes about target_s
        rows = np.linspace(0, w.M - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.gemm_relu_rows(A, B, rows)
        dt = time.perf_counter() - t0
        if dt >= target_s / 2 or n >= w.M:
            break
        n = int(min(w.M, max(n + threads, n * min(8.0, target_s / max(dt, 1e-6)))))
        n = min(w.M, -(-n // threads) * threads)
    flop = 2.0 * n * w.N * w.K
    # and the whole 256^3 problem on one thread (the oracle's result does not
    # depend on the thread count)
    from tiled_dense_gemm_06_amd import workloads as wl

    A1, B1 = wl.make_inputs(wl.WORKLOADS["square256"])
    t1 = time.perf_counter()
    oracle.gemm_relu(A1, B1, threads=1)
    dt1 = time.perf_counter() - t1
    return {
        "value": flop / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle", "cpu": cpu_model(),
        "sample": f"{n} of {w.M} output rows ({n}x{w.N}x{w.K} multiply-adds, all K), {dt:.2f} s wall "
                  f"on {threads} threads",
        "single_thread_square256": {"seconds": dt1, "value": 2.0 * 256 ** 3 / dt1 / 1e12, "unit": "TFLOPS"},
    }


# dense block-scaled MFMA peaks of MI355X (AMD's published dense figures)
PEAK_MX_TFLOPS = {"e4m3": 5000.0, "e5m2": 5000.0, "e2m1": 10100.0}


def mx_cpu_baseline(fmt, w, A, SA, Bt, SB, target_s: float):
    """The block-scaled oracle as it stands, on whole sampled output rows."""
    import numpy as np

    import oracle
    import oracle.mx as omx

    threads = oracle.default_threads()
    n = min(threads, w.M)
    while True:
        rows = np.linspace(0, w.M - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        omx.gemm_relu_mx_rows(fmt, A, SA, Bt, SB, rows)
        dt = time.perf_counter() - t0
        if dt >= target_s / 2 or n >= w.M:
            break
        n = int(min(w.M, max(n + threads, n * min(8.0, target_s / max(dt, 1e-6)))))
        n = min(w.M, -(-n // threads) * threads)
    return {
        "value": 2.0 * n * w.N * w.K / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
        "cpu": cpu_model(),
        "sample": f"{n} of {w.M} output rows ({n}x{w.N}x{w.K} block-scaled multiply-adds, all K), "
                  f"{dt:.2f} s wall on {threads} threads",
    }


def bench_mx(args, torch, tlg, wl, dev) -> int:
    """The block-scaled path (tlg_gemm_relu_mx) on the workload's shape."""
    import numpy as np

    from tiled_dense_gemm_06_amd.profiling import measured_traffic

    fmt = args.mx
    w = wl.WORKLOADS[args.workload]
    if w.K % 128:
        print("bench.py: the block-scaled path needs K % 128 == 0", file=sys.stderr)
        return 2
    A, SA, Bt, SB = wl.make_mx_inputs(fmt, w.M, w.N, w.K, seed=w.seed, kind="random")
    plan = tlg.plan_mx(fmt, w.M, w.N, w.K, config=args.config)
    bits = 4 if fmt == "e2m1" else 8
    alg_bytes = (w.M + w.N) * w.K * bits // 8 + (w.M + w.N) * (w.K // 32) + 2 * w.M * w.N
    R = max(2, math.ceil(2 * MALL_BYTES / alg_bytes) + 1)
    ins = [torch.from_numpy(x).to(dev) for x in (A, SA, Bt, SB)]
    sets = [ins] + [[x.clone() for x in ins] for _ in range(R - 1)]
    Cs = [torch.empty((w.M, w.N), dtype=torch.float16, device=dev) for _ in range(R)]
    h = tlg.handle_for(dev)

    G = args.grouped
    if G and not 2 <= G <= 16:
        print("bench.py: --grouped takes 2 .. 16", file=sys.stderr)
        return 2
    rows = [(w.M * g // G, w.M * (g + 1) // G) for g in range(G)] if G else []
    if G:  # the grouped call picks its tile by the blocks' total tile count
        t256 = sum(-(-(r1 - r0) // 256) * -(-w.N // 256) for r0, r1 in rows)
        gcfg = args.config if args.config >= 0 else (0 if t256 > 128 else 1)
        plan = {"config_name": tlg._native.tlg_plan_mx_config_name(gcfg)}

    def step(i, stream):
        a, sa, b, sb = sets[i % R]
        if G:
            tlg.gemm_relu_mx_grouped(fmt, [a[r0:r1] for r0, r1 in rows], [sa[r0:r1] for r0, r1 in rows], [b] * G,
                                     [sb] * G, [Cs[i % R][r0:r1] for r0, r1 in rows], config=args.config, handle=h,
                                     stream=stream)
        else:
            tlg.gemm_relu_mx(fmt, a, sa, b, sb, out=Cs[i % R], config=args.config, handle=h, stream=stream)

    K = args.steps
    tm = time_steps(torch, step, K, args.warmup, graph=not args.eager)
    wall = tm["wall"]
    ms_per_step = tm["ms_per_step"]
    avg_launch_s = tm["launch_ms_avg"] / 1e3
    tflops = w.flop / (ms_per_step / 1e3) / 1e12
    peak = PEAK_MX_TFLOPS[fmt]
    achieved = w.flop / avg_launch_s / 1e12
    out = {
        "metric": f"block-scaled GEMM+ReLU TFLOPS ({fmt} codes, one E8M0 scale per 32 k, fp32 acc, fp16 out)",
        "value": tflops, "unit": "TFLOPS", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": fmt, "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "seed": w.seed,
                   "inputs": "random codes (exponents bias-3..bias+3, 1 in 16 zero/subnormal), scales 2^-2..2^2",
                   "kernel": plan["config_name"], "grouped": G, "rotated_buffers": R, "alg_bytes": alg_bytes,
                   "timing": tm["timing"],
                   "accumulate": "f32", "epilogue": "relu, round-to-nearest-even to f16"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak,
                     "traffic": measured_traffic(f"{w.name}_mx_{fmt}", plan["config_name"])
                     if args.config < 0 and not G else None,
                     "kernel": plan["config_name"],
                     "launch_ms_avg": avg_launch_s * 1e3, "launch_ms_min": tm["launch_ms_min"]},
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = mx_cpu_baseline(fmt, w, A, SA, Bt, SB, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def copy_calibration(torch, dev, nbytes: int, steps: int, warmup: int) -> int:
    """A plain copy of a known size: reads nbytes and writes nbytes per launch.
    Under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it gives the factor between
    those counters and real HBM bytes."""
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / max(1, steps)
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": steps + warmup,
                      "ms_per_copy": ms, "GB_per_s_read_plus_write": 2 * nbytes / ms / 1e6}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="square8192")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle sample size: about this many seconds of wall time on the host's cores")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the records the default run adds after its timed steps (the skinny workload's "
                         "HBM-bound record and the interleaved vendor-BLAS reference at 8192^3)")
    ap.add_argument("--variant", default="auto",
                    help="kernel family to time (auto = what tlg_gemm_relu picks; others for comparisons): "
                         "auto, tiled_pipe, tiled_dma, tiled_general, splitk, naive")
    ap.add_argument("--config", type=int, default=-1, help="tile configuration index of --variant (-1 = library's choice)")
    ap.add_argument("--splits", type=int, default=0, help="split-K count for --variant splitk (0 = library's choice)")
    ap.add_argument("--trans-b", action="store_true",
                    help="pass B transposed (an N x K row-major copy) through tlg_gemm_relu_bt")
    ap.add_argument("--grouped", type=int, default=0, metavar="G",
                    help="split M into G row blocks (2 <= G <= 16) and run them as one tlg_gemm_relu_grouped "
                         "call (the blocks share B); the work per step is unchanged")
    ap.add_argument("--mx", choices=["e4m3", "e5m2", "e2m1"],
                    help="time the block-scaled path (tlg_gemm_relu_mx) with these element codes instead")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one from the host, each between its own pair of events "
                         "(default: capture them in a HIP graph and time one replay, which removes the host's "
                         "per-call launch cost)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM, time a plain device-to-device copy of MIB MiB (the reference "
                         "kernel for scaling the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "multi-GPU runs are not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tiled_dense_gemm_06_amd as tlg
    from tiled_dense_gemm_06_amd import workloads as wl
    from tiled_dense_gemm_06_amd.profiling import measured_traffic

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration > 0:
        return copy_calibration(torch, dev, args.copy_calibration << 20, args.steps, args.warmup)
    if args.mx:
        return bench_mx(args, torch, tlg, wl, dev)
    w = wl.WORKLOADS[args.workload]
    A, B = wl.make_inputs(w)
    names = {v: k for k, v in tlg._native.VARIANT_NAMES.items()}
    if args.variant not in names:
        print(f"bench.py: unknown variant {args.variant}", file=sys.stderr)
        return 2
    variant = names[args.variant]
    if args.grouped and not 2 <= args.grouped <= 16:
        print("bench.py: --grouped takes 2 .. 16", file=sys.stderr)
        return 2
    if args.grouped and (variant != tlg.TLG_VARIANT_AUTO or args.splits):
        print("bench.py: --grouped takes only --config", file=sys.stderr)
        return 2
    if args.trans_b and (variant not in (tlg.TLG_VARIANT_AUTO, tlg.TLG_VARIANT_TILED_PIPE, tlg.TLG_VARIANT_TILED_DMA,
                                         tlg.TLG_VARIANT_SPLITK) or args.splits):
        print("bench.py: --trans-b takes --variant auto, tiled_pipe, tiled_dma or splitk and --config", file=sys.stderr)
        return 2
    if args.trans_b:
        B = np.ascontiguousarray(B.T)
    if args.grouped:
        # the grouped call picks its tile by the total tile count of the blocks
        rows = [(w.M * g // args.grouped, w.M * (g + 1) // args.grouped) for g in range(args.grouped)]
        # (the library's rule: from 128 tiles of 256 x 256 in total the
        # pipelined 256 x 256 kernel, grouped configuration 4 (16 x 16 x 32
        # MFMA) for K % 64 == 0 and, B not transposed, N % 8 == 0, else 3
        # (32 x 32 x 16); below, direct-to-LDS tiles 0..2 by tile count)
        t256 = sum(-(-(r1 - r0) // 256) * -(-w.N // 256) for r0, r1 in rows)
        t128 = sum(-(-(r1 - r0) // 128) * -(-w.N // 128) for r0, r1 in rows)
        pipe16_ok = w.K % 64 == 0 and (args.trans_b or w.N % 8 == 0)
        gcfg = args.config if args.config >= 0 else ((4 if pipe16_ok else 3) if t256 >= 128 else
                                                     1 if t128 >= 192 else 2)
        name = (tlg.tlg_plan_config_name(tlg.TLG_VARIANT_TILED_PIPE, 17) if gcfg == 4
                else tlg.tlg_plan_config_name(tlg.TLG_VARIANT_TILED_PIPE, 7) if gcfg == 3
                else tlg.tlg_plan_config_name(tlg.TLG_VARIANT_TILED_DMA, gcfg))
        plan = {"config_name": name, "variant_name": "grouped", "splits": 1}
    else:
        plan = tlg.plan(w.M, w.N, w.K, variant=variant, config=args.config, splits=args.splits,
                        trans_b=args.trans_b)

    # Rotate among R copies of the inputs and outputs so the working set is
    # more than twice the Infinity Cache: every step reads from HBM.
    R, As, Bs, Cs = rotated_inputs(torch, w, dev, A, B)
    h = tlg.handle_for(dev)

    def step(i, stream):
        j = i % R
        if args.grouped:
            tlg.gemm_relu_grouped([As[j][r0:r1] for r0, r1 in rows], [Bs[j]] * len(rows),
                                  [Cs[j][r0:r1] for r0, r1 in rows], trans_b=args.trans_b, config=args.config,
                                  handle=h, stream=stream)
        else:
            tlg.gemm_relu(As[j], Bs[j], out=Cs[j], handle=h, stream=stream, variant=variant, config=args.config,
                          splits=args.splits, trans_b=args.trans_b)

    K = args.steps
    tm = time_steps(torch, step, K, args.warmup, graph=not args.eager)
    wall = tm["wall"]
    ms_per_step = tm["ms_per_step"]
    avg_launch_s = tm["launch_ms_avg"] / 1e3

    tflops = w.flop / (ms_per_step / 1e3) / 1e12
    if plan["variant_name"] == "splitk" or w.flop / w.alg_bytes < 314.6:
        achieved = w.alg_bytes / avg_launch_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = w.flop / avg_launch_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_MFMA_TFLOPS}
    plain = args.variant == "auto" and args.config < 0 and not (args.trans_b or args.grouped)
    roof["traffic"] = measured_traffic(w.name, plan["config_name"]) if plain else None
    roof["kernel"] = plan["config_name"]
    roof["launch_ms_avg"] = avg_launch_s * 1e3
    roof["launch_ms_min"] = tm["launch_ms_min"]

    props = torch.cuda.get_device_properties(dev)
    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOPS", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "seed": w.seed, "inputs": w.description,
                   "lda": w.K, "ldb": w.N, "ldc": w.N, "kernel": plan["config_name"],
                   "variant": plan["variant_name"], "splits": plan["splits"], "rotated_buffers": R,
                   "trans_b": bool(args.trans_b), "grouped": args.grouped, "timing": tm["timing"],
                   "accumulate": "f32", "epilogue": "relu, round-to-nearest-even to f16"},
        "roofline": roof,
        "pct_of_fp16_peak": 100.0 * tflops / PEAK_MFMA_TFLOPS,
        "wall_s_timed": wall,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, **gpu_sysfs_info(props)},
    }
    default_run = plain and args.variant == "auto" and not args.eager and not args.no_extras
    if default_run and w.name == "square8192":
        # both outside the timed region above
        out["vendor_reference"] = vendor_reference(torch, tlg, w, As, Bs, Cs, R, rounds=4,
                                                   calls=max(10, min(K, 40)))
    del As, Bs, Cs
    if default_run and w.name != "skinny16x14336x4096":
        torch.cuda.empty_cache()
        out["skinny"] = skinny_record(torch, tlg, wl, dev, steps=max(K, 200), warmup=max(args.warmup, 20))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
