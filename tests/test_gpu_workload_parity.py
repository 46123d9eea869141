"""Full-output parity of the five workloads, in the launch configuration the
benchmark times (the default plan), against the CPU oracle.

For each workload the seeded inputs of its own distribution and the
integer-valued variant from the same seed are run through the C ABI, and
the whole M x N output is compared with the oracle's: bit-exact on integer
inputs (every partial sum is an exact integer in fp32, so no summation order
can change a bit), |got - ref| <= 1e-2 + 4e-3 |ref| elementwise otherwise.
The definition is the quick-start kernel of the TileLang article
(aiwiki.ai/wiki/tilelang, "Programming model").

Each comparison appends one parity record (JSON) to the file named by
TLG_PARITY_LOG (default gpurun_out/parity_records.jsonl under the repository
root): the workload, the kernel, the sha256 of A and B, whether the output
is bit-exact, the number of differing elements, the largest absolute error,
the largest distance in fp16 units in the last place, and the fraction of
elements inside the tolerance.
"""
import json
import os
import time

import numpy as np
import pytest

import oracle
import tiled_dense_gemm_06_amd as tlg
from tiled_dense_gemm_06_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LOG = os.environ.get("TLG_PARITY_LOG", os.path.join(ROOT, "gpurun_out", "parity_records.jsonl"))


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def parity_record(got_bits: np.ndarray, ref_bits: np.ndarray) -> dict:
    """Comparison figures of two fp16 outputs given as uint16 bit patterns."""
    g = got_bits.view(np.float16).astype(np.float64)
    r = ref_bits.view(np.float16).astype(np.float64)
    err = np.abs(g - r)
    tol = 1e-2 + 4e-3 * np.abs(r)
    # non-negative finite fp16 values are ordered like their bit patterns
    ulp = np.abs(got_bits.astype(np.int64) - ref_bits.astype(np.int64))
    diff = got_bits != ref_bits
    return {
        "bit_exact": bool(not diff.any()),
        "mismatches": int(diff.sum()),
        "elements": int(got_bits.size),
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_ulp": int(ulp.max()) if ulp.size else 0,
        "within_tol_frac": float((err <= tol).mean()) if err.size else 1.0,
        "nan": int(np.isnan(g).sum()),
        "negative_or_minus_zero": int(((got_bits & 0x8000) != 0).sum()),
    }


def log_record(rec: dict) -> None:
    os.makedirs(os.path.dirname(LOG), exist_ok=True)
    with open(LOG, "a") as f:
        f.write(json.dumps(rec) + "\n")
    print(json.dumps(rec), flush=True)


@pytest.mark.parametrize("integer", [False, True], ids=["own_distribution", "integer"])
@pytest.mark.parametrize("name", wl.ORDER)
def test_workload_full_output(dev, name, integer):
    w = wl.WORKLOADS[name]
    plan = tlg.plan(w.M, w.N, w.K)
    print(f"parity {name} integer={integer} kernel={plan['config_name']}", flush=True)
    A, B = wl.make_inputs(w, integer=integer)
    Ad = torch.from_numpy(A).to(dev)
    Bd = torch.from_numpy(B).to(dev)
    C = tlg.gemm_relu(Ad, Bd)  # the default plan: what the benchmark launches
    torch.cuda.synchronize()
    got = C.cpu().numpy().view(np.uint16)
    del Ad, Bd, C
    t0 = time.perf_counter()
    ref = oracle.gemm_relu(A, B)
    t_oracle = time.perf_counter() - t0
    rec = {"workload": name, "M": w.M, "N": w.N, "K": w.K,
           "inputs": "integers -2..2 from seed %d" % w.seed if integer else w.description,
           "kernel": plan["config_name"], "variant": plan["variant_name"], "splits": plan.get("splits"),
           "sha256_A": wl.sha256(A), "sha256_B": wl.sha256(B),
           "oracle_s": round(t_oracle, 2), "oracle_threads": oracle.default_threads()}
    rec.update(parity_record(got, ref))
    rec["bar"] = "bit-exact" if integer else "|d| <= 1e-2 + 4e-3|ref|"
    rec["pass"] = rec["bit_exact"] if integer else (rec["within_tol_frac"] == 1.0 and rec["nan"] == 0)
    rec["pass"] = bool(rec["pass"] and rec["negative_or_minus_zero"] == 0)
    log_record(rec)
    assert rec["nan"] == 0 and rec["negative_or_minus_zero"] == 0, rec
    if integer:
        assert rec["bit_exact"], rec
    else:
        assert rec["within_tol_frac"] == 1.0, rec
