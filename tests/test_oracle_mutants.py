"""Each plausible slip planted in a copy of the oracle must fail a pin.

The copies are built from the oracle's C source with one textual change each,
compiled with gcc into a temporary directory, and run through every pin of
oracle_pins.  The real oracle is untouched.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "no_max_subtraction": ("p_row[j] = exp(p_row[j] - m);", "p_row[j] = exp(p_row[j]);"),
    "max_skips_last_key": ("for (int64_t j = 1; j < N; ++j)\n    if (p_row[j] > m)",
                           "for (int64_t j = 1; j < N - 1; ++j)\n    if (p_row[j] > m)"),
    "exp_sign_flipped": ("p_row[j] = exp(p_row[j] - m);", "p_row[j] = exp(m - p_row[j]);"),
    "scale_dropped": ("p_row[j] = scale * dot;", "p_row[j] = dot;"),
    "scale_squared": ("p_row[j] = scale * dot;", "p_row[j] = scale * scale * dot;"),
    "no_normalisation": ("for (int64_t j = 0; j < N; ++j) p_row[j] /= l;", ""),
    "keys_used_as_values": ("o_row[d] += p_row[j] * V[j * D + d];",
                            "o_row[d] += p_row[j] * K[j * D + d];"),
    "dot_drops_last_dim": ("for (int64_t d = 0; d < D; ++d) dot += q_row[d]",
                           "for (int64_t d = 0; d < D - 1; ++d) dot += q_row[d]"),
    "packed_q_v_swapped": ("(((b * N + n) * 3 + which) * H + h) * D + d",
                           "(((b * N + n) * 3 + (2 - which)) * H + h) * D + d"),
    "separate_b_h_swapped": ("((b * H + h) * N + n) * D + d", "((h * B + b) * N + n) * D + d"),
    "output_in_bhnd_order": ("out[((b * N + i) * H + h) * D + d] = o[d];",
                             "out[((b * H + h) * N + i) * D + d] = o[d];"),
    "f16_exponent_bias_off_by_one": ("ldexp(1024.0 + f, e - 25)", "ldexp(1024.0 + f, e - 24)"),
    "f16_subnormal_scale_wrong": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "f16_sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "format_flag_ignored": ("return fmt == 1 ? f16_to_double(bits) : bf16_to_double(bits);",
                            "return bf16_to_double(bits);"),
    "first_key_skipped": ("for (int64_t j = 0; j < N; ++j) {\n    p_row[j] = exp",
                          "p_row[0] = 0.0;\n  for (int64_t j = 1; j < N; ++j) {\n    p_row[j] = exp"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found for {name}"
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib_path = oracle.build(path, os.path.join(tmp_path, "libmutant.so"))
    lib = oracle.load(lib_path)
    failed = []
    for pin_name, pin in oracle_pins.ALL_PINS.items():
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed.append(pin_name)
    assert failed, f"mutant {name} passed every pin"
