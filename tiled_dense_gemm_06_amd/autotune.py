"""Offline tuning sweep for the kernel choice of ``tlg_gemm_relu``.

For each shape of a list (square, rectangular, skinny and ragged classes) it
times every kernel family and tile configuration the library can run on
that shape (forced through ``tlg_gemm_relu_variant``), on synthetic inputs
rotated past the Infinity Cache, and writes the winners that beat the
built-in heuristic by more than a margin as a table compiled into the
library (``csrc/tune_table.inc``). The library consults the table for the
shape's class (ceil(log2) of M, N and K, and whether K or N is ragged)
before its heuristic, and falls back to the heuristic when the tuned choice
cannot serve a problem (e.g. unaligned pointers). The project page
"TileLang: a tile-level DSL for writing GPU kernels in Python" (hysenlabs.com,
"Autotuning, cache behavior and the cost of a search") describes TileLang
preferring a measured search to fixed rules; here the search runs once per
device type, offline, instead of per call.

    python -m tiled_dense_gemm_06_amd.autotune --out tiled_dense_gemm_06_amd/csrc/tune_table.inc

needs a GPU; rebuild the library afterwards.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

SHAPES = [
    # squares
    (512, 512, 512), (1024, 1024, 1024), (2048, 2048, 2048), (3072, 3072, 3072), (4096, 4096, 4096),
    (6144, 6144, 6144), (8192, 8192, 8192), (2560, 2560, 2560), (2816, 2816, 2816),
    # rectangles
    (4096, 14336, 4096), (14336, 4096, 4096), (2048, 8192, 1024), (8192, 2048, 8192), (1024, 4096, 16384),
    (1024, 8192, 4096), (2560, 4096, 4096),
    # skinny M
    (1, 4096, 4096), (16, 14336, 4096), (32, 14336, 4096), (64, 14336, 4096), (16, 4096, 14336),
    (48, 4096, 14336), (16, 2048, 4096), (8, 8192, 8192), (64, 4096, 8192), (48, 1024, 1024), (48, 1024, 1536),
    (64, 1024, 2048),
    (128, 4096, 4096), (256, 8192, 4096),
    # few tiles, long K
    (512, 512, 4096), (256, 256, 16384), (1024, 1024, 8192), (1536, 2048, 4096), (2048, 2048, 8192),
    # ragged
    (3001, 2049, 1537), (1000, 1000, 1000), (777, 555, 333), (5000, 3000, 2000),
]
MARGIN = 0.05  # a tuned entry must beat the heuristic by this fraction


def clog2(x: int) -> int:
    return 0 if x <= 1 else (x - 1).bit_length()


def shape_class(M: int, N: int, K: int) -> tuple:
    return (clog2(M), clog2(N), clog2(K), 1 if (K % 8 or N % 8) else 0)


def candidates(tlg, M, N, K):
    """(variant, config, splits) triples the library accepts for this shape."""
    out = []
    trials = [(tlg.TLG_VARIANT_AUTO, -1, 0)]
    trials += [(tlg.TLG_VARIANT_TILED_PIPE, c, 0) for c in range(28)]
    trials += [(tlg.TLG_VARIANT_TILED_DMA, c, 0) for c in range(5)]
    if M <= 64:
        # two-kernel split-K (0, 1), stream-K tiles (2), strips with 1..8
        # parts (3), the other strip shapes (4..8), the 64-row strip (9),
        # stream-K strips (10, 11)
        trials += [(tlg.TLG_VARIANT_SPLITK, 3, s) for s in (1, 2, 4, 8)]
        trials += [(tlg.TLG_VARIANT_SPLITK, c, 0) for c in (0, 1, 2) + tuple(range(4, 12))]
    elif K >= 2048:
        # the two-kernel split over 32 x 128 tiles with 2..16 parts
        trials += [(tlg.TLG_VARIANT_SPLITK, 0, s) for s in (0, 2, 4, 8, 16)]
    for v, c, s in trials:
        try:
            p = tlg.plan(M, N, K, variant=v, config=c, splits=s)
        except tlg.TlgError:
            continue
        out.append((v, c, s, p["variant"], p["config"], p["config_name"]))
    return out


def time_call(torch, tlg, As, Bs, Cs, v, c, s, iters=20, replays=5):
    """Average time of one call (us): ``iters`` calls over the rotated buffers
    are captured in a HIP graph, so that small shapes are timed without the
    Python launch overhead, and the graph is replayed ``replays`` times."""
    R = len(As)
    for i in range(3):  # eager warm-up (also creates the handle outside the capture)
        tlg.gemm_relu(As[i % R], Bs[i % R], out=Cs[i % R], variant=v, config=c, splits=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            tlg.gemm_relu(As[i % R], Bs[i % R], out=Cs[i % R], variant=v, config=c, splits=s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (iters * replays) * 1e3


def sweep(shapes, log=print):
    import torch

    import tiled_dense_gemm_06_amd as tlg

    dev = torch.device("cuda:0")
    results = []
    for M, N, K in shapes:
        per = 2 * (M * K + K * N + M * N)
        R = max(2, min(64, math.ceil(2 * (256 << 20) / per) + 1))
        g = torch.Generator(device=dev).manual_seed(M * 131 + N * 17 + K)
        A0 = (torch.rand((M, K), device=dev, generator=g) * 2 - 1).half()
        B0 = (torch.rand((K, N), device=dev, generator=g) * 2 - 1).half()
        As = [A0] + [A0.clone() for _ in range(R - 1)]
        Bs = [B0] + [B0.clone() for _ in range(R - 1)]
        Cs = [torch.empty((M, N), device=dev, dtype=torch.float16) for _ in range(R)]
        rows = []
        cands = candidates(tlg, M, N, K)
        for v, c, s, pv, pc, name in cands:
            us = time_call(torch, tlg, As, Bs, Cs, v, c, s)
            rows.append({"variant": pv, "config": pc, "splits": s, "name": name, "us": us, "auto": v == 0})
        # the heuristic's choice once more at the end (the first timing of a
        # shape pays for the cold start); its better time counts
        auto = next(r for r in rows if r["auto"])
        auto["us"] = min(auto["us"], time_call(torch, tlg, As, Bs, Cs, 0, -1, 0))
        auto_plan = tlg.plan(M, N, K)
        # forced runs of the heuristic's own choice are not a different choice
        others = [r for r in rows if not r["auto"] and not (
            r["variant"] == auto_plan["variant"] and r["config"] == auto_plan["config"]
            and r["splits"] in (0, auto_plan["splits"]))]
        best = min(others, key=lambda r: r["us"]) if others else auto
        results.append({"shape": [M, N, K], "class": list(shape_class(M, N, K)), "auto": auto, "best": best,
                        "auto_splits": auto_plan["splits"],
                        "all": rows})
        log(f"{M}x{N}x{K}: auto {auto['name']} {auto['us']:.1f} us, best {best['name']} (splits {best['splits']}) "
            f"{best['us']:.1f} us")
        del As, Bs, Cs
        torch.cuda.empty_cache()
    return results


def class_groups(results):
    """Measured shapes grouped by their shape class, in measurement order."""
    groups = {}
    for r in results:
        groups.setdefault(tuple(r["class"]), []).append(r)
    return groups


def class_choice(rs):
    """The entry for one class: among the choices that differ from the
    heuristic's on some shape of the class, the (variant, config, splits)
    with the least total time over the class's measured shapes, kept if that
    total beats the heuristic's by MARGIN and no shape of the class runs more
    than 2 % slower than with the heuristic; else None. The heuristic's time
    on a shape is the best of its own timing and forced runs of the same
    choice. Returns (key, name, total us, heuristic total us)."""
    def key(row):
        return (row["variant"], row["config"], row["splits"])

    def same(r, k):  # k is what the heuristic runs on shape r
        return (r["auto"]["variant"], r["auto"]["config"]) == k[:2] and k[2] in (0, r.get("auto_splits", 0))

    base = [min([r["auto"]["us"]] + [x["us"] for x in r["all"] if not x["auto"] and same(r, key(x))]) for r in rs]
    common = None
    for r in rs:
        ks = {key(x) for x in r["all"] if not x["auto"]}
        common = ks if common is None else common & ks
    best = None
    for k in sorted(common or ()):
        if all(same(r, k) for r in rs):
            continue
        us = [min(x["us"] for x in r["all"] if not x["auto"] and key(x) == k) for r in rs]
        if best is None or sum(us) < best[1]:
            best = (k, sum(us), us)
    if best is None:
        return None
    k, total, us = best
    if total > sum(base) * (1 - MARGIN) or any(u > b * 1.02 for u, b in zip(us, base)):
        return None
    name = next(x["name"] for x in rs[0]["all"] if key(x) == k)
    return k, name, total, sum(base)


_ENTRY = re.compile(r"^\s*\{(-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+)\},")


def previous_entries(path: str) -> list:
    """(class, (variant, config, splits), line) of each entry of an existing table."""
    out = []
    if not path or not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            m = _ENTRY.match(line)
            if m:
                v = [int(x) for x in m.groups()]
                if v[0] >= 0:
                    out.append((tuple(v[:4]), tuple(v[4:]), line.rstrip("\n")))
    return out


def table_text(results, device: str, previous=()) -> str:
    lines = ["// Tuned kernel choices by shape class, written by",
             "//   python -m tiled_dense_gemm_06_amd.autotune",
             f"// on {device}. Class: ceil(log2) of M, N, K and whether K or N is not a",
             f"// multiple of 8. An entry is kept when it beat the heuristic by more than {MARGIN:.0%};",
             "// each comment gives the measured shape and both times. Entries of the previous",
             "// table stay while their kernel is still the one chosen for their class.",
             "static const TuneEntry kTuneTable[] = {"]
    n = 0
    new_classes = set()
    for cls, rs in class_groups(results).items():
        pick = class_choice(rs)
        if pick is None:
            continue
        new_classes.add(cls)
        key, name, ours, theirs = pick
        first = "x".join(map(str, rs[0]["shape"]))
        more = "".join(f", {'x'.join(map(str, r['shape']))}" for r in rs[1:])
        lines.append(f"    {{{cls[0]}, {cls[1]}, {cls[2]}, {cls[3]}, {key[0]}, {key[1]}, {key[2]}}},"
                     f"  // {first}: {name} {ours:.1f} us vs {rs[0]['auto']['name']} {theirs:.1f} us"
                     + (f" (totals over {first}{more})" if more else ""))
        n += 1
    # The sweep runs against the library as built, so a class the table
    # already serves measures the tuned kernel as "the heuristic". Such an
    # entry stays (with its original measurement) while its kernel is still
    # what the library ran on every measured shape of the class and no new
    # entry replaced it.
    groups = class_groups(results)
    for cls, key, line in previous:
        rs = groups.get(cls, [])
        if cls in new_classes or not rs:
            continue
        if all((r["auto"]["variant"], r["auto"]["config"]) == key[:2] for r in rs):
            lines.append(line)
            n += 1
    if n == 0:
        lines.append("    {-1, -1, -1, -1, 0, -1, 0},  // no shape beat the heuristic by the margin")
    lines.append("};")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", required=True, help="the table to write (csrc/tune_table.inc)")
    ap.add_argument("--json", help="also write every timing here")
    ap.add_argument("--quick", action="store_true", help="the first four shapes only")
    ap.add_argument("--previous", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc",
                                                       "tune_table.inc"),
                    help="the table the library was built with (its entries are kept while still chosen)")
    ap.add_argument("--from-json", help="no sweep: write the table from the timings a sweep saved with --json")
    args = ap.parse_args()
    previous = previous_entries(args.previous)
    if args.from_json:
        with open(args.from_json) as f:
            saved = json.load(f)
        text = table_text(saved["results"], saved["device"], previous)
        with open(args.out, "w") as f:
            f.write(text)
        return 0
    import torch

    shapes = SHAPES[:4] if args.quick else SHAPES
    t0 = time.time()
    res = sweep(shapes, log=lambda s: print(s, flush=True))
    name = torch.cuda.get_device_properties(0).gcnArchName.split(":")[0]
    device = f"{name}, {len(shapes)} shapes, {time.time() - t0:.0f} s"
    text = table_text(res, device, previous)
    with open(args.out, "w") as f:
        f.write(text)
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"device": device, "results": res}, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
