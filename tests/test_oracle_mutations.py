"""The pins must catch plausible mistakes in the oracle.

Each case copies oracle.c, plants one mistake by a text substitution, builds
the copy on the CPU, and runs the fast oracle pin tests against it in a
subprocess (ORACLE_LIB selects the library).  Every mutant must make at
least one pin fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "ties_away_from_zero": ("nearbyint(a / q)", "round(a / q)"),
    "no_saturation": ("a = F->maxval;                      /* saturation */", "(void)0;"),
    "sign_dropped": ("return (uint8_t)(sign | (field_e << F->mbits) | field_m);",
                     "return (uint8_t)((field_e << F->mbits) | field_m);"),
    "e5m2_bias_16": ("{ 5, 2, 15, 57344.0 }", "{ 5, 2, 16, 57344.0 }"),
    "fp8_subnormal_exponent": ("v = ldexp((double)m, 1 - F->bias - F->mbits);",
                               "v = ldexp((double)m, -F->bias - F->mbits);"),
    "f16_subnormal_exponent": ("v = ldexp((double)m, -14 - 10);", "v = ldexp((double)m, -15 - 10);"),
    "unscale_divides": ("float y = orc_f16_to_f32(g[i]) * inv;", "float y = orc_f16_to_f32(g[i]) / S;"),
    "check_inputs_not_outputs": ("if (!isfinite(y))\n                any = 1;",
                                 "if (!isfinite(orc_f16_to_f32(g[i])))\n                any = 1;"),
    "no_canonical_nan": ("o[i] = f32_of_bits(CANONICAL_NAN);", "o[i] = y;"),
    "growth_strict_gt": ("if (*tracker >= interval)", "if (*tracker > interval)"),
    "tracker_kept_on_skip": ("*tracker = 0;\n        if (skips)", "if (skips)"),
    "flag_not_cleared": ("            *tracker = 0;\n        }\n    }\n    *found_inf = 0;\n}",
                         "            *tracker = 0;\n        }\n    }\n}"),
    "amax_counts_inf": ("if (isfinite(f) && fabsf(f) > amax)", "if (!isnan(f) && fabsf(f) > amax)"),
    "no_floor": ("float a = amax > floor_ ? amax : floor_;", "float a = amax; (void)floor_;"),
    "scale_inverted": ("return a / (float)fmt_max(fmt);", "return (float)fmt_max(fmt) / a;"),
    "multiply_by_reciprocal": ("float y = f / s;", "float y = f * (1.0f / s);"),
    "dequant_block_transposed": ("(r / br) * nbc + c / bc;", "(c / bc) * nbc + r / br;"),
    "delayed_latest_only": ("        if (history[i] > hmax)", "        if (i == p && history[i] > hmax)"),
    "delayed_ring_stuck": ("    *pos = (p + 1) % hlen;", "    *pos = p;"),
    "delayed_uses_new_scale": ("    *scale_used = s;", "    *scale_used = *scale_state * 2.0f;"),
    "sumsq_wrong_unit": ("uint64_t G = (uint64_t)(fabs(g) * 16777216.0);", "uint64_t G = (uint64_t)(fabs(g) * 8388608.0);"),
    "sumsq_not_accumulated": ("    total += X;", "    total = X;"),
    "norm_without_inverse": ("*norm_sq = (d * 0x1p-48) * ((double)inv * (double)inv);", "*norm_sq = (d * 0x1p-48);"),
    "hyst_consecutive_inverted": ("        if (consecutive)\n            *h = H;",
                                  "        if (!consecutive)\n            *h = H;"),
    "hyst_no_min_scale": ("*S = lowered > min_scale ? lowered : min_scale;", "*S = lowered;"),
    "hyst_no_refill_at_growth": ("            if (!consecutive)\n                *h = H;",
                                 "            (void)consecutive;"),
    "hyst_budget_off_by_one": ("if (*h <= 1) {", "if (*h <= 0) {"),
    "hyst_window_not_restarted": ("        *tracker = 0;\n        if (*h <= 1) {",
                                  "        if (*h <= 1) {"),
    "mx_scale_rounded_down": ("return (float)(m == 0.5 ? ldexp(1.0, e - 1) : ldexp(1.0, e));",
                              "return (float)ldexp(1.0, e - 1);"),
    "mx_byte_bias_128": ("(uint8_t)(e - 1 + 127)", "(uint8_t)(e - 1 + 128)"),
    "block_1x32_as_1x64": ("{ *br = 1; *bc = 32; }", "{ *br = 1; *bc = 64; }"),
    "mx_nan_byte_ignored": ("b == 0xFF ? f32_of_bits(CANONICAL_NAN) : ", ""),
    "nan_input_unsigned": ("return (uint8_t)((signbit(f) ? 0x80 : 0x00) | 0x7F);", "return 0x7F;"),
    "bf16_ties_away": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))",
                       "if (dropped >= 0x8000u)"),
    "bf16_truncates": ("        ++kept;\n    return (uint16_t)kept;", "    return (uint16_t)kept;"),
}

FAST_PINS = ["tests/test_oracle_formats.py", "tests/test_oracle_unscale.py",
             "tests/test_oracle_quant.py", "tests/test_oracle_delayed.py",
             "tests/test_oracle_sumsq.py", "tests/test_oracle_hysteresis.py",
             "tests/test_oracle_mx.py", "tests/test_oracle_bf16.py"]


def _run_mutant(name, tmp_dir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    if src.count(old) != 1:
        return "mutation anchor not unique/absent: %r" % old
    mut = os.path.join(tmp_dir, "oracle_%s.c" % name)
    with open(mut, "w") as fh:
        fh.write(src.replace(old, new))
    so = os.path.join(tmp_dir, "liboracle_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                    "-fPIC", "-shared", "-w", "-o", so, mut, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not slow and not gpu",
                        "-p", "no:cacheprovider", *FAST_PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    if r.returncode == 0:
        return "mutant %s survived every pin:\n%s" % (name, r.stdout[-2000:])
    return None


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Build and test every mutant, several at a time."""
    from concurrent.futures import ThreadPoolExecutor
    tmp = str(tmp_path_factory.mktemp("mutants"))
    names = sorted(MUTANTS)
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        return dict(zip(names, ex.map(lambda n: _run_mutant(n, tmp), names)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_results):
    assert mutant_results[name] is None, mutant_results[name]
