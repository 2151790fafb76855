"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a textual edit of ``oracle/arfuse_oracle.c`` compiled into a
temporary library on the CPU; the committed oracle is never modified. This
shows the pins in ``oracle_pins.py`` are sensitive to the kinds of error a
reader would worry about: a wrong summation order or width, a misplaced eps,
a wrong index, a wrong rounding tie rule, a wrong bit layout.
"""

import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "arfuse_oracle.c")

E4M3_TIE = ("    double dist = fabs(ax - oracle_e4m3_value((uint8_t)c));\n"
            "    if (dist < bestd || (dist == bestd && (c & 1) == 0 && (best & 1) == 1)) {")
E2M1_TIE = ("    double dist = fabs(aq - kE2M1[c]);\n"
            "    if (dist < bestd || (dist == bestd && (c & 1) == 0 && (best & 1) == 1)) {")

MUTANTS = {
    "residual_added_first": [
        ("float acc = oracle_bf16_to_f32(partials[0][e]);",
         "float acc = oracle_bf16_to_f32(residual[e]) + oracle_bf16_to_f32(partials[0][e]);"),
        ("h[e] = acc + oracle_bf16_to_f32(residual[e]);", "h[e] = acc;")],
    "double_accumulator": [
        ("float acc = oracle_bf16_to_f32(partials[0][e]);",
         "double acc = oracle_bf16_to_f32(partials[0][e]);")],
    "reverse_rank_order": [
        ("float acc = oracle_bf16_to_f32(partials[0][e]);",
         "float acc = oracle_bf16_to_f32(partials[n - 1][e]);"),
        ("for (int i = 1; i < n; ++i) acc = acc + oracle_bf16_to_f32(partials[i][e]);",
         "for (int i = n - 2; i >= 0; --i) acc = acc + oracle_bf16_to_f32(partials[i][e]);")],
    "eps_outside_sqrt": [
        ("double inv = 1.0 / sqrt(ms + (double)eps);",
         "double inv = 1.0 / (sqrt(ms) + (double)eps);")],
    "mean_over_d_minus_1": [
        ("double ms = ss / (double)d;", "double ms = ss / (double)(d > 1 ? d - 1 : 1);")],
    "float_sum_of_squares": [("double ss = 0.0;", "float ss = 0.0f;")],
    "gamma_reversed": [("* (double)gamma[j]);", "* (double)gamma[d - 1 - j]);")],
    "gamma_dropped": [(" * (double)gamma[j]);", ");")],
    "normalize_bf16_h": [
        ("    oracle_rmsnorm_rows(h, gamma, eps, 1, d, y);",
         "    for (int64_t j = 0; j < d; ++j) h[j] = oracle_bf16_to_f32(oracle_bf16_rne(h[j]));\n"
         "    oracle_rmsnorm_rows(h, gamma, eps, 1, d, y);")],
    "bf16_ties_away": [("pick = ((lo >> 16) & 1u) ? hi : lo;", "pick = hi;")],
    "bf16_truncate": [("  if (dlo < dhi)\n    pick = lo;", "  if (1)\n    pick = lo;")],
    "e4m3_ties_down": [(E4M3_TIE, E4M3_TIE.replace(
        "dist < bestd || (dist == bestd && (c & 1) == 0 && (best & 1) == 1)", "dist < bestd"))],
    "e4m3_no_saturation_guard": [("  if (ax > 448.0) return 0x7E;\n", "")],
    "e4m3_subnormal_exponent": [("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)")],
    "e2m1_ties_down": [(E2M1_TIE, E2M1_TIE.replace(
        "dist < bestd || (dist == bestd && (c & 1) == 0 && (best & 1) == 1)", "dist < bestd"))],
    "e2m1_table_typo": [("{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}",
                         "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0}")],
    "scale_by_reciprocal": [("float ratio = bm / 6.0f;", "float ratio = bm * (1.0f / 6.0f);")],
    "codes_by_reciprocal": [("mag = oracle_e2m1_rne(fabsf(y[j]) / s);",
                             "mag = oracle_e2m1_rne(fabsf(y[j]) * (1.0f / s));")],
    "nibbles_swapped": [("(uint8_t)(c16[2 * k] | (c16[2 * k + 1] << 4))",
                         "(uint8_t)(c16[2 * k + 1] | (c16[2 * k] << 4))")],
    "sign_dropped": [("code16[j] = (uint8_t)((signbit(y[j]) ? 8u : 0u) | mag);",
                      "code16[j] = mag;")],
    "sign_of_zero_lost": [("(signbit(y[j]) ? 8u : 0u)", "(y[j] < 0.0f ? 8u : 0u)")],
    "block_max_signed": [("float a = fabsf(y[j]);", "float a = y[j];")],
    "zero_scale_not_special": [("if (s != 0.0f) mag = oracle_e2m1_rne", "mag = oracle_e2m1_rne")],
    "fp8_sign_dropped": [("out[e] = (uint8_t)((signbit(q) ? 0x80u : 0u) | oracle_e4m3_rne(fabsf(q)));",
                          "out[e] = (uint8_t)oracle_e4m3_rne(fabsf(q));")],
    "fp8_scale_divides": [("float q = y[e] * inv_scale;", "float q = y[e] / inv_scale;")],
    "no_residual_adds_zero_first": [
        ("        float acc = oracle_bf16_to_f32(prow[0][j]);\n        for (int i = 1; i < n; ++i)",
         "        float acc = 0.0f + oracle_bf16_to_f32(prow[0][j]);\n        for (int i = 1; i < n; ++i)")],
    "sentinel_counted_per_element": [("    pending += hit;", "    for (int k = 0; k < 8; ++k) pending += part[8 * v + k] == sentinel;")],
    "ll_flag_misread": [("flag = (flag << 8) | p[8 + k];", "flag = (flag << 8) | p[7 + k];")],
    "ll_payload_bytes_swapped": [
        ("(uint16_t)(p[2 * k] | ((uint16_t)p[2 * k + 1] << 8))",
         "(uint16_t)(p[2 * k + 1] | ((uint16_t)p[2 * k] << 8))")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, "mutation anchor not unique/present: %r" % old
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = oracle.build(out=str(tmp_path / "libmutant.so"), src=str(path),
                       extra_flags=["-Wno-unused-parameter", "-Wno-unused-variable"])
    orc = oracle.Oracle(oracle.load(lib))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, ZeroDivisionError) as e:
            failed.append((pin.__name__, str(e)[:80]))
            break
    assert failed, "mutant %s passed every pin" % name


# Planted mistakes in the chained replay (Python, oracle/__init__.py): each
# replaces Oracle.chain with a plausible wrong version and must fail a pin.
def _chain_residual_not_handed_on(self, sets, r0, gamma, eps, k, fp4=False, per_call=False):
    return [self.allreduce_rmsnorm(sets[c] if per_call else sets, r0, gamma, eps, fp4=fp4)
            for c in range(k)]


def _chain_sets_reversed(self, sets, r0, gamma, eps, k, fp4=False, per_call=False):
    res, out = r0, []
    for c in range(k):
        r = self.allreduce_rmsnorm(sets[k - 1 - c] if per_call else sets, res, gamma, eps, fp4=fp4)
        out.append(r)
        res = r["residual_out"]
    return out


def _chain_first_set_only(self, sets, r0, gamma, eps, k, fp4=False, per_call=False):
    res, out = r0, []
    for c in range(k):
        r = self.allreduce_rmsnorm(sets[0] if per_call else sets, res, gamma, eps, fp4=fp4)
        out.append(r)
        res = r["residual_out"]
    return out


def _chain_one_call_short(self, sets, r0, gamma, eps, k, fp4=False, per_call=False):
    res, out = r0, []
    for c in range(k):
        r = self.allreduce_rmsnorm(sets[c] if per_call else sets, res, gamma, eps, fp4=fp4)
        out.append(r)
        if c + 1 < k - 1:
            res = r["residual_out"]
    return out


CHAIN_MUTANTS = {"residual_not_handed_on": _chain_residual_not_handed_on,
                 "sets_reversed": _chain_sets_reversed,
                 "first_set_only": _chain_first_set_only,
                 "last_hand_off_missing": _chain_one_call_short}


@pytest.mark.parametrize("name", sorted(CHAIN_MUTANTS))
def test_chain_mutant_fails_a_pin(name):
    broken = type("BrokenChain", (oracle.Oracle,), {"chain": CHAIN_MUTANTS[name]})()
    with pytest.raises(AssertionError):
        oracle_pins.pin_chain(broken)
