"""HBM traffic of a kernel from rocprofv3 counters, for the benchmark's roofline record.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report KiB per
dispatch. Those counters do not read true bytes on every part, so they are
scaled by what the same counters read for a plain device-to-device copy of a
known size (``bench.py --copy-calibration MIB``): factor = copy bytes /
counter bytes, separately for reads and writes.

Usage (after the counter runs, on the CSV files rocprofv3 wrote)::

    python -m tiled_dense_gemm_06_amd.profiling traffic --workload square8192 \\
        --kernel k_tiled_pipe --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-mib 512

It records, under the digest of the library's kernel sources, the scaled
fetch and write bytes per launch in ``profiles/traffic.json``; ``bench.py``
reports them only while the kernel sources still have that digest.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_KERNEL = "copyBuffer"


def kernel_sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + [os.path.join(ROOT, "include", "tlg.h")]


def kernel_source_digest() -> str:
    """sha256 over every source the kernels are built from."""
    h = hashlib.sha256()
    for p in kernel_sources():
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
    digest = kernel_source_digest()
    if data.get("kernel_source_sha256") != digest:
        data = {"kernel_source_sha256": digest, "workloads": {}}
    data["calibration"] = {"copy_bytes": copy_bytes, "fetch_factor": fetch_factor, "write_factor": write_factor}
    rec = {"kernel": args.kernel, "fetch_bytes": fetch, "write_bytes": write, "bytes_per_launch": fetch + write}
    data["workloads"][args.workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def measured_traffic(workload: str):
    """Scaled HBM bytes per launch for a workload, if taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_sha256") != kernel_source_digest():
        return None
    rec = data.get("workloads", {}).get(workload)
    return None if not rec else rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--kernel", required=True, help="substring of the kernel name")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    args = ap.parse_args()
    print(json.dumps(traffic(args)))


if __name__ == "__main__":
    main()
