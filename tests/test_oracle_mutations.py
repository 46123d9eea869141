"""Planted mistakes: each test compiles a copy of the oracle with one
plausible bug (a dropped term, a wrong sign, a swapped index, a wrong
rounding rule) and checks that the pins catch it. The mutants live in a
temporary directory on the CPU; nothing here touches a GPU."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, mutated text)
MUTATIONS = [
    ("dropped_last_k_term", "for (int64_t k = 0; k < jb->K; k++) {",
     "for (int64_t k = 0; k + 1 < jb->K; k++) {"),
    ("relu_wrong_sign", "return (acc > 0.0f) ? acc : 0.0f;", "return (acc < 0.0f) ? -acc : 0.0f;"),
    ("relu_missing", "return (acc > 0.0f) ? acc : 0.0f;", "return acc;"),
    ("a_transposed", "float a = oracle_f16_to_f32(jb->A[i * jb->lda + k]);",
     "float a = oracle_f16_to_f32(jb->A[k * jb->lda + i]);"),
    ("b_transposed", "Bf[k * N + j] = oracle_f16_to_f32(B[k * ldb + j]);",
     "Bf[k * N + j] = oracle_f16_to_f32(B[j * ldb + k]);"),
    ("ties_not_even", "if (rem > half || (rem == half && (q & 1u))) q += 1u;",
     "if (rem >= half) q += 1u;"),
    ("truncating_cast", "if (rem > half || (rem == half && (q & 1u))) q += 1u;", "(void)half;"),
    ("subnormal_widening", "e -= 1;", "e -= 2;"),
    ("exponent_bias", "return bits_to_f32(sign | ((exp - 15u + 127u) << 23) | (frac << 13));",
     "return bits_to_f32(sign | ((exp - 16u + 127u) << 23) | (frac << 13));"),
]

# The quick pins run against every mutant (full pins take longer).
QUICK = ("worked_examples or ones_closed_form or k1_products or tiny_brute_force "
         "or identity or rank_one or integer_exactness_all_shapes and square256 "
         "or f16_to_f32_exhaustive or golden_cases or sums_exercise_rne")


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique or missing: {name}"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(mutant_c), "-o", str(so)], check=True)
    env = dict(os.environ, TLG_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", QUICK],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"


# ---------------------------------------------------------------- the block-scaled oracle

MX_SRC = os.path.join(ROOT, "oracle", "oracle_mx.c")

# (The order of the two E2M1 codes inside a byte is not among them: A and B
# share it, so swapping it pairs the same elements and leaves every sum, and
# every result, unchanged; a byte never straddles a 32-element block.)
MX_MUTATIONS = [
    ("scale_bias", "return ldexp(1.0, (int)e - 127);", "return ldexp(1.0, (int)e - 128);"),
    ("scale_of_neighbour_block", "oracle_mx_scale(SA[i * ldsa + b])",
     "oracle_mx_scale(SA[i * ldsa + (b ^ 1) % (K / 32)])"),
    ("last_element_of_block_dropped", "k < 32 * b + 32; k++", "k < 32 * b + 31; k++"),
    ("e4m3_bias", "return minifloat(code, 4, 3, 7);", "return minifloat(code, 4, 3, 8);"),
    ("e5m2_bias", "return minifloat(code, 5, 2, 15);", "return minifloat(code, 5, 2, 16);"),
    ("e2m1_bias", "return minifloat(code & 0xfu, 2, 1, 1);", "return minifloat(code & 0xfu, 2, 1, 0);"),
    ("subnormal_exponent", "v = ldexp((double)f, 1 - bias - mb);", "v = ldexp((double)f, -bias - mb);"),
    ("sign_ignored", "return sign ? -v : v;", "return v;"),
    ("relu_missing", "static double relu64(double x) { return (x > 0.0) ? x : 0.0; }",
     "static double relu64(double x) { return x; }"),
    ("ties_away", "if (rem > half || (rem == half && (q & 1ull))) q += 1ull;", "if (rem >= half) q += 1ull;"),
]


@pytest.mark.parametrize("name,old,new", MX_MUTATIONS, ids=[m[0] for m in MX_MUTATIONS])
def test_mx_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(MX_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique or missing: {name}"
    mutant_c = tmp_path / "oracle_mx_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / f"liboracle_mx_{name}.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(mutant_c), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, TLG_ORACLE_MX_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_mx_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"


# ---------------------------------------------------------------- the layout and batching wrappers
# Broken copies of oracle.gemm_relu_bt, oracle.gemm_relu_grouped and
# oracle.mx.gemm_relu_mx_grouped, each with one plausible bookkeeping mistake;
# the wrapper pins must reject every one.

from test_oracle_wrapper_pins import check_bt, check_grouped, check_mx_grouped  # noqa: E402

import numpy as np  # noqa: E402

import oracle.mx as omx  # noqa: E402


def _bt_dropped_transpose(A, Bt, threads=None):
    return oracle.gemm_relu(A, np.ascontiguousarray(Bt), threads)


def _bt_a_for_b(A, Bt, threads=None):
    # B taken from A's buffer (operands mixed up): right shape when M == N
    return oracle.gemm_relu(A, np.ascontiguousarray(A.T if A.shape[0] == Bt.shape[0] else Bt.T), threads)


def _grouped_reversed(problems, trans_b=False, threads=None):
    return list(reversed(oracle.gemm_relu_grouped(problems, trans_b, threads)))


def _grouped_ignores_trans_b(problems, trans_b=False, threads=None):
    return [oracle.gemm_relu(A, B, threads) for A, B in problems]


def _grouped_b_of_next_problem(problems, trans_b=False, threads=None):
    f = oracle.gemm_relu_bt if trans_b else oracle.gemm_relu
    out = []
    for t, (A, _) in enumerate(problems):
        B = problems[(t + 1) % len(problems)][1]
        out.append(f(A, B, threads))
    return out


def _mx_grouped_rotated(fmt, problems, threads=None):
    res = omx.gemm_relu_mx_grouped(fmt, problems, threads)
    return res[1:] + res[:1]


def _mx_grouped_scales_of_next(fmt, problems, threads=None):
    out = []
    for t, (A, SA, Bt, SB) in enumerate(problems):
        SAn, SBn = problems[(t + 1) % len(problems)][1], problems[(t + 1) % len(problems)][3]
        if SAn.shape != SA.shape or SBn.shape != SB.shape:
            SAn, SBn = SA, SB[::-1].copy()
        out.append(omx.gemm_relu_mx(fmt, A, SAn, Bt, SBn, threads))
    return out


@pytest.mark.parametrize("mutant", [_bt_dropped_transpose, _bt_a_for_b], ids=lambda f: f.__name__)
def test_bt_pin_catches_planted_mistake(mutant):
    with pytest.raises((AssertionError, ValueError)):
        check_bt(mutant)


@pytest.mark.parametrize("mutant", [_grouped_reversed, _grouped_ignores_trans_b, _grouped_b_of_next_problem],
                         ids=lambda f: f.__name__)
def test_grouped_pin_catches_planted_mistake(mutant):
    with pytest.raises((AssertionError, ValueError)):
        check_grouped(mutant)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("mutant", [_mx_grouped_rotated, _mx_grouped_scales_of_next], ids=lambda f: f.__name__)
def test_mx_grouped_pin_catches_planted_mistake(mutant, fmt):
    pytest.importorskip("torch")
    with pytest.raises((AssertionError, ValueError)):
        check_mx_grouped(mutant, fmt)
