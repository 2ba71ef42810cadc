"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each.

Every mutant is one textual edit of oracle.c (a swapped nibble, a dropped ReLU,
a wrong exponent bias, a reversed tie-break, ...), compiled into a temporary
library; the pin suite (tests/test_oracle_pins.py) then runs against it in a
subprocess and must fail.  CPU only; the real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "nibble_order": ("return (d & 1) ? (b >> 4) : (b & 15);", "return (d & 1) ? (b & 15) : (b >> 4);"),
    "no_relu": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    "relu_keeps_nan": ("double relu = dot > 0.0 ? dot : 0.0;",
                       "double relu = (dot > 0.0 || isnan(dot)) ? dot : 0.0;"),
    "nan_logit_kept": ("    if (isnan(acc))\n        return -INFINITY;\n", ""),
    "e2m1_subnormal": ("(e == 0) ? 0.5 * m", "(e == 0) ? 1.0 * m"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "ue8m0_bias": ("return ldexp(1.0, b - 127);", "return ldexp(1.0, b - 128);"),
    "e4m3_bias": ("mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    "tie_toward_higher": ("return (x->t > y->t) - (x->t < y->t);", "return (x->t < y->t) - (x->t > y->t);"),
    "scale_block_shift": ("orc_ue8m0(s[d / 32]);", "orc_ue8m0(s[(d / 32 + 1) % (D / 32)]);"),
    "one_weight_for_all_heads": ("acc += w[h] * relu;", "acc += w[0] * relu;"),
    "duplicates_kept": ("if (m == 0 || ids_out[i] != ids_out[m - 1])", "if (1)"),
    "ks_ignored": ("        if (lo < ks)\n            lo = ks;\n        if (hi > ke)\n            hi = ke;\n        for",
                   "        if (hi > ke)\n            hi = ke;\n        for"),
    "fp8_rowscale_dropped": ("            dot *= rowscale;", "            dot *= 1.0;"),
    "q_row_stride": ("q_values ? q_values + (int64_t)r * H * (D / 2) : NULL",
                     "q_values ? q_values + (int64_t)r * (D / 2) : NULL"),
    "slot_reversed": ("    int slot = t % kv->page_size;", "    int slot = kv->page_size - 1 - t % kv->page_size;"),
    "no_minus_one_fill": ("        out[i] = -1;", "        out[i] = 0;"),
    "output_unsorted": ("    qsort(out, count, sizeof(int32_t), cmp_i32);\n", ""),
    "last_head_dropped": ("    for (int h = 0; h < H; h++) {\n        double dot", "    for (int h = 0; h < H - (H > 1); h++) {\n        double dot"),
    "expand_end_counts_blocks": ("                valid += (int32_t)(hi - lo);", "                valid += (int32_t)sbk;"),
    # the bf16 scoring variant
    "bf16_truncates": ("if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0))", "if (0)"),
    "bf16_ties_away": ("if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0))", "if (frac >= 0.5)"),
    "bf16_rounds_through_fp32": ("return (float)orc_round_bf16(acc);", "return (float)orc_round_bf16((float)acc);"),
    "bf16_logits_not_rounded": ("return (float)orc_round_bf16(acc);", "return (float)acc;"),
    "bf16_exponent_bias": ("mag = ldexp(1.0 + m / 128.0, e - 127);", "mag = ldexp(1.0 + m / 128.0, e - 128);"),
    "bf16_weight_mantissa_dropped": ("orc_bf16(((const uint16_t *)weights)[(int64_t)r * H + h])",
                                     "orc_bf16(((const uint16_t *)weights)[(int64_t)r * H + h] & 0xFF80)"),
    "bf16_subnormal_spacing": ("    if (lsb < -133)\n        lsb = -133;", "    if (lsb < -126)\n        lsb = -126;"),
    # the candidate-source layer
    "source_sum_pooling": ("                if (!any || lg > best)\n                    best = lg;",
                           "                best = any ? best + lg : lg;"),
    "source_ties_toward_higher_block": ("    return (x->b > y->b) - (x->b < y->b);",
                                        "    return (x->b < y->b) - (x->b > y->b);"),
    "source_ks_ignored": ("            if (lo < ks)\n                lo = ks;\n            if (hi > ke)\n                hi = ke;\n            float best",
                          "            if (hi > ke)\n                hi = ke;\n            float best"),
    "source_partial_block_past_ke": ("            if (lo < ks)\n                lo = ks;\n            if (hi > ke)\n                hi = ke;\n            float best",
                                     "            if (lo < ks)\n                lo = ks;\n            float best"),
    "source_publishes_by_score_order": ("            out[j] = blk[j].b;\n        emit_ascending(out, count, nb);",
                                        "            out[j] = blk[j].b;\n        for (int32_t j = count; j < nb; j++)\n            out[j] = -1;"),
    "bf16_no_overflow": ("    if (v >= ldexp(1.0, 128))\n        v = INFINITY;\n", ""),
}


def _run_pins(tmp_path, source):
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(source)
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(lib), str(mutant), "-lm"])
    env = dict(os.environ, IDX_ORACLE_MUTANT_LIB=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    proc = _run_pins(tmp_path, open(SRC).read())
    assert proc.returncode == 0, proc.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    proc = _run_pins(tmp_path, src.replace(old, new))
    # exit code 1: tests ran and at least one failed (not a collection error)
    assert proc.returncode == 1, f"mutant {name}: rc={proc.returncode}\n{proc.stdout[-2000:]}"
