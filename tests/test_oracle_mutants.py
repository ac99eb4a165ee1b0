"""Plant plausible mistakes in copies of the C oracle (CPU only) and check
that the pins in test_oracle.py catch every one of them."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
from tests import test_oracle as T

SRC = open(oracle_build.SRC).read()

# (name, original text, mistaken text)
MUTANTS = [
    ("drop_logit", "y = y * (p->logit ? p->logit[i] : 1.0f);", ""),
    ("drop_pertoken", "y = y * (p->pertoken_scale ? p->pertoken_scale[p->pertoken_per_tensor ? 0 : i] : 1.0f);", ""),
    ("per_tensor_scale_ignored", "p->pertoken_scale[p->pertoken_per_tensor ? 0 : i]",
     "(p->pertoken_per_tensor ? 1.0f : p->pertoken_scale[i])"),
    ("scale_ignores_expert", "return ((const float*)p->scale)[g * p->n + j];",
     "return ((const float*)p->scale)[j];"),
    ("nibble_high_first", "(word >> (4 * (j % 8)))", "(word >> (4 * (7 - j % 8)))"),
    ("nibble_unsigned", "return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    ("transposed_weight", "return (int32_t)w[(g * p->k + kk) * p->n + j];",
     "return (int32_t)w[(g * p->n + j) * p->k + kk];"),
    ("counts_read_as_cumulative", "start[g] = prev;\n      end[g] = prev + v;",
     "start[g] = prev;\n      end[g] = v > prev ? v : prev;"),
    ("group_start_off_by_one", "if (v < prev) return ORC_ERR_GROUPLIST;\n      start[g] = prev;",
     "if (v < prev) return ORC_ERR_GROUPLIST;\n      start[g] = prev + (prev > 0);"),
    ("seed_off_by_one", "d >= p->shared_input_offset && d < p->shared_input_offset + p->bsdp",
     "d > p->shared_input_offset && d <= p->shared_input_offset + p->bsdp"),
    ("combine_descending", "for (int64_t i = 0; i < m; ++i) {\n      if (group_of[i] < 0) continue;",
     "for (int64_t i = m - 1; i >= 0; --i) {\n      if (group_of[i] < 0) continue;"),
    ("acc_sign", "acc[j] += a * wrow[j];", "acc[j] -= a * wrow[j];"),
    ("one_rounding_in_double", "float y = (float)acc;             /* int32 -> fp32, round to nearest even */",
     "double yd = (double)acc * scale_at(p, g, j) * (p->pertoken_scale ? p->pertoken_scale[i] : 1.0f)"
     " * (p->logit ? p->logit[i] : 1.0f); return (float)yd; float y = 0;"),
]

PINS = [
    lambda: [T.test_worked_example_pertoken_matmul(g) for g in (0, 1)],
    T.test_combine_from_worked_example,
    T.test_int4_nibble_decoding,
    T.test_acc_closed_form_extremes,
    T.test_group_list_types_agree,
    T.test_empty_groups_contribute_nothing,
    T.test_zero_activations_give_the_seed,
    T.test_int4_equals_int8_with_small_values,
    T.test_rounding_error_within_bound,
    T.test_per_tensor_scale_is_every_rows_scale,
    lambda: [T.test_brute_force_matches_oracle(c) for c in T._tiny_cases()[:40]],
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant, tmp_path):
    name, old, new = mutant
    assert SRC.count(old) == 1, f"mutation site for {name} not unique/present"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    lib_path = tmp_path / "libmutant.so"
    inc = os.path.dirname(oracle_build.SRC)
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-I", inc, str(src), "-o", str(lib_path)], check=True)
    lib = ctypes.CDLL(str(lib_path))
    for fn in ("orc_gmm_finalize_routing", "orc_out_rows", "orc_acc_rows", "orc_group_ranges"):
        getattr(lib, fn).restype = ctypes.c_int
    saved = oracle._lib
    oracle._lib = lib
    caught = []
    try:
        for i, pin in enumerate(PINS):
            try:
                pin()
            except (AssertionError, oracle.OracleError, ValueError):
                caught.append(i)
                break
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught the planted mistake {name}"
