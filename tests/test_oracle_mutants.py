"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in a copy of oracle/ep_oracle.c (a dropped
term, a wrong sign, index or bound, a wrong rounding rule), builds it with the
oracle's own gcc flags into a temporary library, and runs the pin battery
against it through ``oracle.use_library`` in a child process (a mistake that
sends a slot out of range can corrupt memory; the child keeps that away from
the test run).  Every planted mistake must make at least one pin fail, or make
the child die.  The mutants live only in a temporary directory.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)
if os.path.dirname(HERE) not in sys.path:
    sys.path.insert(0, os.path.dirname(HERE))

import oracle
import test_oracle_dedup as pins_dd
import test_oracle_dispatch_combine as pins_dc
import test_oracle_mx_f16 as pins_mx
import test_oracle_formats as pins_fmt
import test_oracle_layout as pins_lay
import test_oracle_scales_mn as pins_mn
import test_oracle_variants as pins_var

SRC = os.path.join(os.path.dirname(oracle.__file__), "ep_oracle.c")

MUTANTS = [
    ("E4M3 ties go up", "else code = (lo % 2 == 0) ? lo : lo + 1;", "else code = lo + 1;"),
    ("E4M3 loses the sign of zero", "uint8_t sign = signbit(v) ? 0x80 : 0x00;",
     "uint8_t sign = (v < 0) ? 0x80 : 0x00;"),
    ("E4M3 subnormal spacing", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("E4M3 exponent bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("bf16 ties away from zero", "double r = nearbyint(n);", "double r = floor(n + 0.5);"),
    ("bf16 rounds through fp32 first", "double n = a / quantum;",
     "double n = (double)(float)a / quantum;"),
    ("bf16 subnormal quantum", "quantum = ldexp(1.0, -133);", "quantum = ldexp(1.0, -134);"),
    ("slot uses the next expert's offset", "slot_idx[p] = expert_offsets[e] + r;",
     "slot_idx[p] = expert_offsets[e + 1] + r;"),
    ("slot rank starts at 1", "int32_t r = cursor[e]++;", "int32_t r = ++cursor[e];"),
    ("capacity bound off by one", "if (cap > 0 && r >= cap)", "if (cap > 0 && r > cap)"),
    ("unrouted -1 counted as an error", "if (e == -1) continue;                        /* R2: unrouted */",
     ""),
    ("group ranges overlap", "e < (g + 1) * per_group; ++e) s +=",
     "e <= (g + 1) * per_group && e < E; ++e) s +="),
    ("slots filled in reverse pair order",
     "for (int64_t p = 0; p < P; ++p) {\n        int64_t e = topk_idx[p];\n        if (e < 0 || e >= E) { slot_idx[p] = -1;",
     "for (int64_t p = P - 1; p >= 0; --p) {\n        int64_t e = topk_idx[p];\n        if (e < 0 || e >= E) { slot_idx[p] = -1;"),
    ("offsets as an inclusive scan", "expert_offsets[0] = 0;\n", "expert_offsets[0] = num_tokens_per_expert[0];\n"),
    ("dispatch reads the wrong token", "int64_t t = p / k;", "int64_t t = p % k;"),
    ("no floor under tiny blocks", "float a = amax > 1e-4f ? amax : 1e-4f;", "float a = amax;"),
    ("scale inverted", "float scale = a / 448.0f;", "float scale = 448.0f / a;"),
    ("amax of signed values", "float m = fabsf(bf16_to_float(x_row[c]));", "float m = bf16_to_float(x_row[c]);"),
    ("E4M3 NaN keeps its sign", "if (isnan(v)) return 0x7F;", "if (isnan(v)) return signbit(v) ? 0xFF : 0x7F;"),
    ("block maximum takes NaN", "if (m > amax) amax = m;\n        }\n        float a = amax > 1e-4f",
     "if (!(m <= amax)) amax = m;\n        }\n        float a = amax > 1e-4f"),
    ("FP8 copies take the wrong scale row", "memcpy(recv_scales + (int64_t)s * nb, sc,",
     "memcpy(recv_scales + (int64_t)(s / 2) * nb, sc,"),
    ("combine uses the first weight only", "acc += (double)w[t * k + j] *", "acc += (double)w[t * k] *"),
    ("combine sums in fp32", "double acc = 0.0;", "float acc = 0.0f;"),
    ("combine drops the last pair", "for (int32_t j = 0; j < k; ++j) {\n            int32_t s = slot_idx[t * k + j];\n            if (s < 0) continue;\n            acc",
     "for (int32_t j = 0; j < k - 1; ++j) {\n            int32_t s = slot_idx[t * k + j];\n            if (s < 0) continue;\n            acc"),
    ("dequant reads the wrong block scale", "(double)scales[r * nb + c / 128]", "(double)scales[r * nb + c % nb]"),
    ("power-of-two scale one step too large", "while (ldexp(448.0, e) < (double)a) ++e;",
     "while (ldexp(448.0, e) <= (double)a) ++e;"),
    ("power-of-two rescale multiplies", "double v = ldexp((double)bf16_to_float(x_row[c]), -e);",
     "double v = ldexp((double)bf16_to_float(x_row[c]), e);"),
    ("FP8 combine reads block 0's scale", "(double)scales[(int64_t)s * nb + c / 128];",
     "(double)scales[(int64_t)s * nb];"),
    ("FP8 combine forgets the weight", "acc += (double)w[t * k + j] * ep_oracle_e4m3_decode(",
     "acc += ep_oracle_e4m3_decode("),
    ("dedup groups listed in descending order",
     "for (int32_t g = 0; g < G; ++g)\n            if (in_group[t * G + g]) group_idx[t * kg + i++] = g;",
     "for (int32_t g = G - 1; g >= 0; --g)\n            if (in_group[t * G + g]) group_idx[t * kg + i++] = g;"),
    ("dedup group of an expert by modulo", "in_group[t * G + e / per_group] = 1;",
     "in_group[t * G + e % G] = 1;"),
    ("dedup counts pairs instead of tokens", "in_group[t * G + e / per_group] = 1;",
     "in_group[t * G + e / per_group] += 1;"),
    ("dedup rows start one row late", "int32_t row = group_offsets[g] + cursor[g]++;",
     "int32_t row = group_offsets[g] + ++cursor[g];"),
    ("dedup receiver keeps other groups' experts", "int mine = e >= 0 && e < E && e / per_group == g;",
     "int mine = e >= 0 && e < E;"),
    ("dedup receiver weights not masked", "mine ? topk_weights[t * k + j] : 0.0f",
     "topk_weights[t * k + j]"),
    ("MX shared exponent one too high", "se = (e - 1) - 8;", "se = e - 8;"),
    ("MX uses 7 as E4M3's largest exponent", "se = (e - 1) - 8;", "se = (e - 1) - 7;"),
    ("MX shared exponent not clamped below", "if (se < -127) se = -127;\n            if (se > 127)",
     "if (se > 127)"),
    ("MX amax of signed values", "double m = fabs(ep_oracle_bf16_to_double(x_row[c]));",
     "double m = ep_oracle_bf16_to_double(x_row[c]);"),
    ("MX dequant scale bias off by one", "double x = ldexp(1.0, (int)b - 127);", "double x = ldexp(1.0, (int)b - 128);"),
    ("fp16 ties away from zero", "double r = nearbyint(a / quantum) * quantum;",
     "double r = floor(a / quantum + 0.5) * quantum;"),
    ("fp16 overflows at the largest finite value", "if (r > 65504.0)", "if (r >= 65504.0)"),
    ("fp16 subnormal spacing", "quantum = ldexp(1.0, -24);           /* subnormal spacing",
     "quantum = ldexp(1.0, -25);           /* subnormal spacing"),
    ("fp16 decode exponent bias", "ldexp(1024.0 + m, e - 15 - 10)", "ldexp(1024.0 + m, e - 14 - 10)"),
    ("fp16 combine forgets the weight", "acc += (double)w[t * k + j] * ep_oracle_f16_to_double(",
     "acc += ep_oracle_f16_to_double("),
    ("token-in-group matrix copied short", "memcpy(is_token_in_group, in_group, (size_t)T * (size_t)G);",
     "memcpy(is_token_in_group, in_group, (size_t)T);"),
    ("MX combine scale bias off by one", "return b == 255 ? NAN : ldexp(1.0, (int)b - 127);",
     "return b == 255 ? NAN : ldexp(1.0, (int)b - 128);"),
    ("MX combine decodes scale byte 0 as zero", "return b == 255 ? NAN : ldexp(1.0, (int)b - 127);",
     "return b == 255 ? NAN : (b == 0 ? 0.0 : ldexp(1.0, (int)b - 127));"),
    ("MX dequant decodes the NaN byte as 2^128", "if (b == 255) { y[r * H + c] = 0x7FC0u; continue; }", ""),
    ("MX combine reads the 128-channel block's scale", "e8m0_value(scales[(int64_t)s * nb + c / 32]);",
     "e8m0_value(scales[(int64_t)s * nb + c / 128]);"),
    ("MN-major layout indexed row-major", "memcpy(dst + ((int64_t)c * rows + r) * entry_bytes,",
     "memcpy(dst + (r * entries + c) * entry_bytes,"),
    ("group combine drops the last group",
     "for (int32_t i = 0; i < kg; ++i) {\n            int32_t r = group_slot[t * kg + i];",
     "for (int32_t i = 0; i < kg - 1; ++i) {\n            int32_t r = group_slot[t * kg + i];"),
]


def _battery():
    """Fast pins (the exhaustive FP8 sweep is left out; the fixtures and the
    torch comparison on structured values cover the same rules)."""
    checks = [
        pins_fmt.test_e4m3_golden_values,
        pins_fmt.test_e4m3_decode_table_is_the_format,
        pins_fmt.test_e4m3_matches_torch_decode,
        pins_fmt.test_bf16_golden_values,
        pins_fmt.test_bf16_rounding_from_binary64_exact,
        pins_lay.test_layout_golden,
        pins_lay.test_layout_random_with_masks_and_overflow,
        pins_lay.test_layout_empty_and_degenerate,
        pins_dc.test_fp8_block_golden,
        pins_dc.test_fp8_dispatch_copies_and_rows,
        pins_dc.test_fp8_zero_and_signed_zero_blocks,
        pins_dc.test_fp8_nonfinite_block_golden,
        pins_dc.test_bf16_dispatch_is_the_gather,
        pins_dc.test_bf16_dispatch_padded_skips_dropped,
        pins_dc.test_combine_golden,
        pins_dc.test_combine_one_hot_is_a_gather,
        pins_dc.test_combine_vs_float64_sum_and_order,
        pins_dc.test_combine_all_skipped_gives_positive_zero,
        pins_dc.test_fp8_round_trip_error_bound_through_combine,
    ]
    checks += [lambda s=s: pins_lay.test_layout_brute_force_tiny(s) for s in range(12)]
    checks += [lambda: pins_dc.test_fp8_quantisation_properties("dsv3", 8)]
    checks += [lambda: pins_dc.test_combine_identity_round_trip("tiny")]
    checks += [pins_var.test_pow2_golden_blocks, pins_var.test_combine_fp8_golden,
               pins_var.test_combine_fp8_one_hot_is_the_dequantisation,
               pins_var.test_combine_fp8_vs_float64_sum,
               lambda: pins_var.test_pow2_scale_is_the_smallest_power_of_two("dsv3")]
    checks += [pins_dd.test_group_layout_golden, pins_dd.test_combine_groups_golden,
               pins_dd.test_one_group_and_one_group_per_expert,
               pins_dd.test_combine_groups_is_the_unit_weight_combine,
               lambda: pins_dd.test_group_layout_matches_a_stable_sort("dsv3"),
               lambda: pins_dd.test_second_level_layout_is_the_expert_layout("lowlat"),
               lambda: pins_dd.test_receiver_metadata_partitions_each_token("dsv3"),
               lambda: pins_dd.test_dedup_round_trip("tiny")]
    checks += [lambda s=s: pins_dd.test_group_layout_brute_force_tiny(s) for s in range(8)]
    checks += [pins_mx.test_mxfp8_golden_blocks, pins_mx.test_mxfp8_error_bound_and_saturation,
               pins_mx.test_mxfp8_dispatch_and_dequant,
               lambda: pins_mx.test_mxfp8_shared_exponent_and_codes("dsv3"),
               pins_mx.test_f16_golden_values, pins_mx.test_f16_rounding_against_numpy,
               pins_mx.test_combine_f16_golden,
               pins_mx.test_combine_f16_one_hot_is_a_gather_and_round_trip_is_exact,
               pins_mx.test_combine_f16_is_the_rounded_exact_sum,
               pins_mx.test_combine_mxfp8_golden, pins_mx.test_combine_mxfp8_one_hot_is_the_dequantisation,
               pins_mx.test_combine_mxfp8_vs_float64_sum, pins_mx.test_combine_mxfp8_extreme_scale_bytes,
               pins_mx.test_combine_mxfp8_nan_scale_and_codes, pins_mx.test_dequant_mxfp8_extreme_scale_bytes]
    checks += [lambda: pins_mn.test_scales_mn_major_matches_index_loops(3, 5),
               lambda: pins_mn.test_scales_mn_major_matches_index_loops(17, 56),
               lambda: pins_mn.test_mn_major_columns_are_the_tokens_scales(False)]
    return checks


def test_unmutated_oracle_passes_the_battery():
    for check in _battery():
        check()


def _run_battery_on(lib_path: str) -> int:
    """Number of pins that fail against the library at lib_path."""
    failures = 0
    with oracle.use_library(lib_path):
        for check in _battery():
            try:
                check()
            except Exception:  # an assertion, or a shape / status error
                failures += 1
    return failures


def _build_and_run(tmp_dir, i, old, new):
    # the first occurrence is the site (a few lines recur in the variant
    # functions further down, which have mutants of their own)
    src = open(SRC).read()
    assert old in src, "mutation site not found: %r" % old
    mutated = os.path.join(tmp_dir, "mutant%d.c" % i)
    with open(mutated, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = os.path.join(tmp_dir, "libmutant%d.so" % i)
    subprocess.run(["gcc", *oracle.GCC_FLAGS, mutated, "-o", lib, "-lm"], check=True)
    r = subprocess.run([sys.executable, os.path.abspath(__file__), lib], capture_output=True,
                       text=True, timeout=300)
    return r.returncode, r.stdout[-400:] + r.stderr[-400:]


def test_planted_mistakes_are_caught(tmp_path):
    # the child itself must pass on the real oracle, or every mutant would look caught
    r = subprocess.run([sys.executable, os.path.abspath(__file__), oracle.build()],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-400:] + r.stderr[-400:]
    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(lambda im: _build_and_run(str(tmp_path), im[0], im[1][1], im[1][2]),
                              enumerate(MUTANTS)))
    survivors = [MUTANTS[i][0] for i, (rc, _) in enumerate(results) if rc == 0]
    assert not survivors, "planted mistakes that passed every pin: %s" % survivors


if __name__ == "__main__":
    # child process: exit status 0 means every pin passed against this library
    n = _run_battery_on(sys.argv[1])
    print("failing pins:", n)
    sys.exit(1 if n else 0)
