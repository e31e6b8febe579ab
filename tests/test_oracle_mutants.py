"""The oracle pins must catch plausible slips in the oracle.

Each case copies oracle/bitlinear_oracle.c, plants one mistake on the CPU
(a dropped abs, a wrong divisor, truncation instead of round-half-even, a
missing epsilon, a wrong tie-break, a misplaced bit, a transposed operand, a
wrong clamp, a wrong activation constant, a slip in the ReLU^2 gate, the
RMSNorm, the a4.8 outlier split or the 2:4 trit code), builds it, and runs the pin suite
against it: the suite must fail for every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bitlinear_oracle.c")

MUTANTS = {
    "abs_dropped": ("row += fabs((double)w);", "row += (double)w;"),
    "divisor_N": ("double mean = total / (double)(N * K);", "double mean = total / (double)(N);"),
    "no_eps": ("float d = beta + 1e-5f;", "float d = beta;"),
    "trunc_not_rne_w": ("float r = rintf(W[i] / d);", "float r = truncf(W[i] / d);"),
    "round_half_away_w": ("float r = rintf(W[i] / d);", "float r = roundf(W[i] / d);"),
    "tie_to_higher_k": ("if (best < 0 || mag > best_mag) { best = i;", "if (best < 0 || mag >= best_mag) { best = i;"),
    "rank_signed": ("float mag = fabsf(w[i]);", "float mag = w[i];"),
    "bit_position": ("int bit = 8 * (j % 4) + 2 * (j / 4);", "int bit = 2 * j;"),
    "code_offset": ("put_code(out + r * (K / 4), k, (unsigned)(v + 1));",
                    "put_code(out + r * (K / 4), k, (unsigned)(1 - v));"),
    "act_const_128": ("float s = 127.0f / (g * up);", "float s = 128.0f / (g * up);"),
    "act_round_half_away": ("float v = rintf((x[k] * up) * s);", "float v = roundf((x[k] * up) * s);"),
    "act_order": ("float v = rintf((x[k] * up) * s);", "float v = rintf((x[k] * 127.0f) / g);"),
    "act_no_tiny_row_scaling": ("const float up = (g < 0x1p-100f) ? 0x1p100f : 1.0f;", "const float up = 1.0f;"),
    "xscale_inverse": ("x_scale[r] = g / 127.0f;", "x_scale[r] = 127.0f / g;"),
    "transposed_w": ("s += (int64_t)q[m * K + k] * (int64_t)w_eff[n * K + k];",
                     "s += (int64_t)q[m * K + k] * (int64_t)w_eff[k * N + n];"),
    "nm_mask_nibble_order": ("masks[r * mrow + g / 2] |= (uint8_t)(mask << (4 * (g % 2)));",
                             "masks[r * mrow + g / 2] |= (uint8_t)(mask << (4 * (1 - g % 2)));"),
    "nm_keep_one_less": ("for (int round = 0; round < n; ++round)", "for (int round = 1; round < n; ++round)"),
    "gate_no_relu": ("float relu = x[k] > 0.0f ? x[k] : 0.0f;", "float relu = x[k];"),
    "gate_no_square": ("float sq = relu * relu;", "float sq = relu;"),
    "gate_up_dropped": ("v[k] = sq * up[r * K + k];", "v[k] = sq;"),
    "rms_eps_outside_sqrt": ("rinv = 1.0 / sqrt(ss / (double)K + (double)eps);",
                             "rinv = 1.0 / (sqrt(ss / (double)K) + (double)eps);"),
    "rms_sum_not_mean": ("rinv = 1.0 / sqrt(ss / (double)K + (double)eps);",
                         "rinv = 1.0 / sqrt(ss + (double)eps);"),
    "rms_gamma_dropped": ("for (int64_t k = 0; k < K; ++k) v[k] = v[k] * gamma[k];",
                          "for (int64_t k = 0; k < K; ++k) v[k] = v[k] * 1.0f;"),
    "rms_scale_without_rinv": ("x_scale[r] = (g == 0.0f) ? 0.0f : (float)((double)g / 127.0 * rinv);",
                               "x_scale[r] = (g == 0.0f) ? 0.0f : (float)((double)g / 127.0);"),
    "rms_after_gamma": ("for (int64_t k = 0; k < K; ++k) ss += (double)v[k] * (double)v[k];",
                        "for (int64_t k = 0; k < K; ++k) ss += (double)v[k] * (double)v[k] * (double)gamma[k] * (double)gamma[k];"),
    "had_butterfly_sign": ("v[i] = a + c;\n                    v[i + h] = a - c;",
                           "v[i] = a - c;\n                    v[i + h] = a + c;"),
    "had_skip_first_stage": ("for (int64_t h = 1; h < B; h *= 2)", "for (int64_t h = 2; h < B; h *= 2)"),
    # the H-BitLinear's block quantiser sits one level deeper than a4.8's
    # 4-bit part, which has lines of the same text: anchor by indentation
    "h4_const_8": ("\n            float s = 7.0f / (g * pre);", "\n            float s = 8.0f / (g * pre);"),
    "h4_no_tiny_row_scaling": ("\n            const float pre = (g < 0x1p-100f) ? 0x1p100f : 1.0f;",
                               "\n            const float pre = 1.0f;"),
    "h4_scale_unnormalised": ("x_scale[r] = (float)((double)g / 7.0 / sqrt((double)B));",
                              "x_scale[r] = (float)((double)g / 7.0);"),
    "h4_trunc": ("\n                float c = rintf((v[k] * pre) * s);", "\n                float c = truncf((v[k] * pre) * s);"),
    "a48_tie_to_higher_k": ("if (best < 0 || mag > best_mag) {\n                    best = k;",
                            "if (best < 0 || mag >= best_mag) {\n                    best = k;"),
    "a48_rank_signed": ("float mag = fabsf(x[k]);", "float mag = x[k];"),
    "a48_one_less": ("for (int64_t round = 0; round < T; ++round)", "for (int64_t round = 1; round < T; ++round)"),
    "a48_lo_keeps_outliers": ("lo[k] = taken[k] ? 0.0f : x[k];", "lo[k] = x[k];"),
    "a48_lo_const_8": ("float s = 7.0f / (g * pre);\n        for (int64_t k = 0; k < K; ++k) {\n            float c",
                       "float s = 8.0f / (g * pre);\n        for (int64_t k = 0; k < K; ++k) {\n            float c"),
    "a48_lo_scale": ("*x_scale = g / 7.0f;", "*x_scale = g / 8.0f;"),
    "a48_rows_swapped": ("rc = oracle_quant_act(hi, 1, K, 0, q + (2 * r) * K, x_scale + 2 * r, rowsum ? rowsum + 2 * r : NULL);",
                         "rc = oracle_quant_act(hi, 1, K, 0, q + (2 * r + 1) * K, x_scale + 2 * r, rowsum ? rowsum + 2 * r : NULL);"),
    "trit_pair_order": ("static const int kPairLo[6] = {0, 0, 0, 1, 1, 2};\nstatic const int kPairHi[6] = {1, 2, 3, 2, 3, 3};",
                        "static const int kPairLo[6] = {0, 0, 1, 0, 1, 2};\nstatic const int kPairHi[6] = {1, 2, 2, 3, 3, 3};"),
    "trit_value_order": ("unsigned code = (unsigned)(9 * p + 3 * (v0 + 1) + (v1 + 1));",
                         "unsigned code = (unsigned)(9 * p + (v0 + 1) + 3 * (v1 + 1));"),
    "trit_bit_stride": ("int64_t bit = (g / 16) * 96 + 6 * (g % 16);\n            for (int b = 0; b < 6; ++b)\n                if (code",
                        "int64_t bit = (g / 16) * 96 + 6 * (g % 15);\n            for (int b = 0; b < 6; ++b)\n                if (code"),
    "trit_string_stride": ("int64_t bit = (g / 16) * 96 + 6 * (g % 16);\n            for (int b = 0; b < 6; ++b)\n                if (code",
                           "int64_t bit = (g / 16) * 90 + 6 * (g % 16);\n            for (int b = 0; b < 6; ++b)\n                if (code"),
    "trit_unpack_swapped": ("w_eff[r * K + 4 * g + kPairLo[p]] = (int8_t)(v / 3 - 1);\n            w_eff[r * K + 4 * g + kPairHi[p]] = (int8_t)(v % 3 - 1);",
                            "w_eff[r * K + 4 * g + kPairLo[p]] = (int8_t)(v % 3 - 1);\n            w_eff[r * K + 4 * g + kPairHi[p]] = (int8_t)(v / 3 - 1);"),
    "epilogue_no_beta": ("Y[m * N + n] = (double)s * (double)beta * (double)x_scale[m];",
                         "Y[m * N + n] = (double)s * (double)x_scale[m];"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % old
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                           "-shared", "-o", str(lib), str(mut), "-lm"])
    env = dict(os.environ, BITLINEAR_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
