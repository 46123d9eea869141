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
