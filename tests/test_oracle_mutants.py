"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a temporary copy of the oracle's C source
(a dropped term, a wrong index, a wrong sign, a wrong exponent bias, the
wrong tie rule, a wrong scale constant or a missing floor), builds it with gcc, swaps it in for the real library and
checks that at least one pin test fails.  Everything runs on the CPU.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_decode_round as T1
from tests import test_oracle_gemm as T2
from tests import test_oracle_quantize as T3
from tests._cases import golden_cases

MUTANTS = {
    "dropped_last_term_of_group": ("for (int64_t k = k0; k < k1; ++k)", "for (int64_t k = k0; k + 1 < k1; ++k)"),
    "a_scale_always_group0": ("(double)a_s[m * G + g]", "(double)a_s[m * G]"),
    "b_scale_always_block0": ("(double)b_s[(n / ORACLE_GROUP) * G + g]", "(double)b_s[g]"),
    "b_scale_indexed_by_row_mod": ("(double)b_s[(n / ORACLE_GROUP) * G + g]", "(double)b_s[(n % 2 < (N + 127) / 128 ? n % 2 : 0) * G + g]"),
    "wrong_sign_of_fold": ("acc += p * s;", "acc -= p * s;"),
    "subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "exponent_bias": ("(int)e - 7", "(int)e - 8"),
    "ties_away_from_zero": ("nearbyint(x / q)", "round(x / q)"),
    "bf16_precision": ("round_to_format(v, 8, -126, 127)", "round_to_format(v, 9, -126, 127)"),
    "fp16_exponent_bias": ("(unsigned)(E + 15) << 10", "(unsigned)(E + 14) << 10"),
    "encode_ties_away_from_zero": ("nearbyint(ldexp(a, 3 - e))", "round(ldexp(a, 3 - e))"),
    "encode_subnormal_boundary": ("if (a < ldexp(1.0, -6)) {", "if (a < ldexp(1.0, -7)) {"),
    "encode_sign_dropped": ("    return sign | code;\n}", "    return code;\n}"),
    "quantize_scale_447": ("(amax > 1e-12f ? amax : 1e-12f) / 448.0f;\n            a_s[",
                           "(amax > 1e-12f ? amax : 1e-12f) / 447.0f;\n            a_s["),
    "quantize_no_floor": ("(amax > 1e-12f ? amax : 1e-12f) / 448.0f;\n            a_s[", "amax / 448.0f;\n            a_s["),
    "blocks_scale_447": ("(amax > 1e-12f ? amax : 1e-12f) / 448.0f;\n            b_s[",
                         "(amax > 1e-12f ? amax : 1e-12f) / 447.0f;\n            b_s["),
    "quantize_signed_amax": ("fabsf(bf16_value(x[m * K + i]))", "bf16_value(x[m * K + i])"),
    "quantize_scale_group0": ("a_s[m * G + g] = s;", "a_s[m * G] = s;"),
    "blocks_scale_row0": ("b_s[bn * G + g] = s;", "b_s[g] = s;"),
    "blocks_ragged_rows_dropped": ("n1 = n0 + ORACLE_GROUP < N ? n0 + ORACLE_GROUP : N;",
                                   "n1 = n0 + ORACLE_GROUP < N ? n0 + ORACLE_GROUP : n0 + (N - n0) / 2;"),
    "blocks_amax_one_row": ("for (int64_t n = n0; n < n1; ++n)\n                for (int64_t c = c0; c < c1; ++c) {\n                    const float v = fabsf",
                            "for (int64_t n = n0; n < n0 + 1; ++n)\n                for (int64_t c = c0; c < c1; ++c) {\n                    const float v = fabsf"),
}

PINS = [
    T1.test_decode_matches_torch_all_codes,
    T1.test_decode_format_landmarks,
    T1.test_round_fp32_matches_numpy,
    T1.test_round_fp16_matches_numpy,
    T1.test_round_bf16_against_value_set,
    T1.test_round_bf16_is_one_step_from_fp64,
    lambda: [T2.test_handworked_cases(c) for c in golden_cases()],
    lambda: T2.test_brute_force_exact_rational(1, 3, 4, 128),
    lambda: T2.test_brute_force_exact_rational(4, 1, 130, 128),
    T2.test_integer_mode_is_exact,
    lambda: T2.test_matches_numpy_blas_of_dequantised_operands(37, 300, 512),
    T2.test_identity_weight_exposes_every_code,
    T2.test_row_and_column_block_locality,
    T3.test_encode_inverts_decode_on_every_finite_code,
    T3.test_midpoints_round_to_even_code,
    T3.test_saturation_at_448,
    T3.test_quantize_constant_group_maps_to_448,
    T3.test_quantize_zero_groups_keep_sign_and_floor,
    T3.test_quantize_groups_and_scales_are_per_row_and_per_128,
    T3.test_dequantised_within_half_a_step,
    T3.test_blocks_constant_block_maps_to_448,
    T3.test_blocks_scale_is_local_to_its_block,
    T3.test_blocks_ragged_last_block_row,
    T3.test_blocks_dequantised_within_half_a_step,
]


def _build_mutant(tmp, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "fp8bg_oracle.c")).read()
    assert src.count(old) == 1, old
    path = os.path.join(tmp, "m.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp, "m.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    path, "-o", lib, "-lm"], check=True)
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        lib_path = _build_mutant(tmp, old, new)
        real = oracle._load()
        monkeypatch.setattr(oracle, "_LIB_PATH", lib_path)
        monkeypatch.setattr(oracle, "_lib", None)
        oracle._load()
        caught = []
        for pin in PINS:
            try:
                pin()
            except Exception:
                caught.append(getattr(pin, "__name__", "lambda"))
        monkeypatch.setattr(oracle, "_lib", real)
    assert caught, f"no pin caught mutant {name}"
