"""Planted mistakes in copies of the oracle are caught by the pins (CPU only).

Each case edits oracle.c in a temporary copy (a plausible slip: a wrong index, a dropped
scale, an off-by-one bias, truncation instead of rounding, a lost sign), compiles it with
gcc and runs the pins against it: at least one pin must fail. The real oracle is never
modified."""
import os

import pytest

import oracle as oracle_pkg
import pins

MUTATIONS = {
    "b_scale_row_modulo": ("(size_t)(n / 128) * KB + kb", "(size_t)(n % 128 % 2) * KB + kb"),
    "a_scale_transposed": ("a_scale[(size_t)m * KB + kb]", "a_scale[(size_t)kb * M + m]"),
    "scale_dropped": ("acc += p * s;", "acc += p;"),
    "e4m3_bias_off_by_one": ("ldexp((double)(8 + f), e - 10)", "ldexp((double)(8 + f), e - 11)"),
    "e4m3_subnormal_scale": ("ldexp((double)f, -9)", "ldexp((double)f, -10)"),
    "sign_lost": ("return s ? -v : v;", "return v;"),
    "bf16_truncates": ("double r = nearbyint(q);", "double r = floor(q);"),
    "bf16_ties_away": ("double r = nearbyint(q);", "double r = round(q);"),
    "bf16_no_subnormal_clamp": ("e = -126;", "e = e;"),
    "mx_wrong_exponent_bias": ("ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 128)"),
    "mx_a_scale_for_b": ("e8m0_decode(b_e8m0[(size_t)n * G + g])", "e8m0_decode(a_e8m0[(size_t)m * G + g])"),
    "block_boundary": ("k < kb * 128 + 128", "k < kb * 128 + 127"),
    "mx_group_boundary": ("k < g * 32 + 32", "k < g * 32 + 31"),
    "pt_b_scale_by_row": ("(double)a_scale[m] * (double)b_scale[n]", "(double)a_scale[m] * (double)b_scale[m]"),
    "pt_b_scale_dropped": ("dot * ((double)a_scale[m] * (double)b_scale[n])", "dot * (double)a_scale[m]"),
    "quant_scale_447": ("float s = amax / 448.0f;", "float s = amax / 447.0f;"),
    "quant_ties_odd": ("(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    "quant_mx_exponent_loose": ("while (amax > ldexp(448.0, e))", "while (amax >= ldexp(448.0, e))"),
    "quant_zero_group_scale": ("            s = 1.0f;", "            s = 2.0f;"),
    "quant_sign_lost": ("return (uint8_t)(signbit(x) ? (best | 0x80) : best);", "return (uint8_t)best;"),
    "pt_last_k_dropped": ("for (int k = 0; k < K; k++)\n                dot +=", "for (int k = 0; k < K - 1; k++)\n                dot +="),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(oracle_pkg.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new)
    path = os.path.join(tmp_path, "oracle_mutant.c")
    open(path, "w").write(mutated)
    lib = oracle_pkg.build(path, os.path.join(tmp_path, "liboracle_mutant.so"))
    mutant = oracle_pkg.Oracle(lib)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, f"mutation {name} slipped past every pin"
