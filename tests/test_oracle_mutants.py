"""Negative controls for the oracle's pins: plant one plausible mistake at a
time in a copy of ``oracle/oracle.c`` (on the CPU), rebuild, and check that at
least one pin in ``test_oracle.py`` rejects the broken copy."""
import os
import shutil

import pytest

import oracle as oracle_pkg
from oracle import Oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle_pkg.__file__), "oracle.c")

# (name, original text, replacement): each must occur exactly once in oracle.c
MUTANTS = [
    ("drop_last_k_block", "for (int kb = 0; kb < Kb; ++kb) {", "for (int kb = 0; kb < Kb - 1; ++kb) {"),
    ("fnuz_bias", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("lost_sign", "return s ? -mag : mag;", "return mag;"),
    ("sfb_ignores_kb", "double scale = (double)j->sa[kb * j->sa_stride] * (double)sb[kb];",
     "double scale = (double)j->sa[kb * j->sa_stride] * (double)sb[0];"),
    ("sfb_block_64", "const float *sb = j->sfb + (int64_t)(n / ORACLE_NBLOCK) * Kb;",
     "const float *sb = j->sfb + (int64_t)(n / 64 < (j->N + 127) / 128 ? n / 64 : 0) * Kb;"),
    ("sfa_k_major", "        j.sa = p->sfa + r; j.sa_stride = p->M;\n        j.b = p->B; j.sfb = p->sfb;",
     "        j.sa = p->sfa + r * (p->K / 128); j.sa_stride = 1;\n        j.b = p->B; j.sfb = p->sfb;"),
    ("c_ignored", "j->out[n] = acc + (j->c_row ? (double)j->c_row[n] : 0.0);", "j->out[n] = acc;"),
    ("b_transposed", "s += j->dec[ap[k]] * j->dec[bp[k]];",
     "s += j->dec[ap[k]] * j->dec[j->b[(int64_t)(kb * ORACLE_KBLOCK + k) * j->N + n]];"),
    ("contig_group0", "        j.b = p->B + (int64_t)g * p->N * p->K;\n        j.sfb = p->sfb + (int64_t)g * Nb * Kb;",
     "        j.b = p->B;\n        j.sfb = p->sfb;"),
    ("masked_off_by_one", "if (m >= valid) {", "if (m > valid) {"),
    ("bf16_ties_up", "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    ("scale_squared", "acc += scale * s;", "acc += scale * scale * s;"),
    ("ue8m0_bias_128", "return ldexp(1.0, (int)e - 127);", "return ldexp(1.0, (int)e - 128);"),
    ("ue8m0_big_endian", "return (uint8_t)(((uint32_t)word >> (8 * j)) & 0xFFu);",
     "return (uint8_t)(((uint32_t)word >> (8 * (3 - j))) & 0xFFu);"),
    ("ue8m0_sfa_k_major", "int32_t w = packed[(g * W + kb / 4) * M + m];",
     "int32_t w = packed[(g * M + m) * W + kb / 4];"),
    ("fp4_drop_last_k_block", "for (int kb = 0; kb != Kb; ++kb) {", "for (int kb = 0; kb != Kb - 1; ++kb) {"),
    ("fp4_c_ignored", "j->out[n] = (j->c_row ? (double)j->c_row[n] : 0.0) + acc;", "j->out[n] = acc;"),
    ("e2m1_lost_sign", "return s ? -1.0 * mag : mag;", "return mag;"),
    ("e2m1_bias_2", "double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);",
     "double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 2);"),
    ("fp4_nibbles_swapped", "uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 0xF);",
     "uint8_t nib = (k & 1) ? (byte & 0xF) : (byte >> 4);"),
    ("fp4_scale_block_64", "acc += sa * oracle_ue8m0_value(ue8m0_byte(wb, blk)) * s;",
     "acc += sa * oracle_ue8m0_value(ue8m0_byte(wb, blk / 2)) * s;"),
    ("kg_drop_last_k_block", "for (int64_t kb = kb_first; kb < kb_end; ++kb) {",
     "for (int64_t kb = kb_first; kb < kb_end - 1; ++kb) {"),
    ("kg_previous_segment", "const int64_t kb_first = p->k_off[g] / ORACLE_KBLOCK,",
     "const int64_t kb_first = p->k_off[g > 0 ? g - 1 : 0] / ORACLE_KBLOCK,"),
    ("kg_a_k_contiguous", "const double a = p->dec[p->A[k * M + m]];",
     "const double a = p->dec[p->A[m * (int64_t)p->K + k]];"),
    ("kg_sfb_first_block", "const float *sb = p->sfb + kb * (int64_t)N;",
     "const float *sb = p->sfb + kb_first * (int64_t)N;"),
    ("kg_c_ignored", "            out[n] += (double)c_row[n];", "            out[n] += 0.0 * (double)c_row[n];"),
    ("bf16_bias_128", "mag = ldexp(1.0 + (double)m / 128.0, e - 127);", "mag = ldexp(1.0 + (double)m / 128.0, e - 128);"),
    ("bf16_subnormal_scale", "mag = ldexp((double)m, -133);", "mag = ldexp((double)m, -132);"),
    ("bf16_drop_last_k", "            for (int k = 0; k < p->K; ++k)\n                acc += a[k]",
     "            for (int k = 0; k < p->K - 1; ++k)\n                acc += a[k]"),
    ("bf16_lost_sign", "return copysign(mag, s ? -1.0 : 1.0);", "return mag;"),
    # (swapping the nibble order of both operands at once leaves every block sum unchanged;
    # swapping it for A alone is a real mistake)
    ("fp4x4_a_nibbles_swapped", "blk += e2m1_nibble(a_row, k, dec4) * e2m1_nibble(b_row, k, dec4);",
     "blk += e2m1_nibble(a_row, k ^ 1, dec4) * e2m1_nibble(b_row, k, dec4);"),
    ("fp4x4_a_scale_block_64", "const double sa = oracle_ue8m0_value(ue8m0_byte(sa_row[kb], j));",
     "const double sa = oracle_ue8m0_value(ue8m0_byte(sa_row[kb], j / 2));"),
    ("fp4x4_a_scale_ignored", "                total += sa * sb * blk;", "                total += sb * blk;"),
    ("fp4x4_last_block_dropped", "for (int j = 0; j < 4; ++j) {\n                double blk = 0.0;",
     "for (int j = 0; j < 3; ++j) {\n                double blk = 0.0;"),
    ("bf16_c_ignored", "out[n] = acc + (p->C ? (double)p->C[r * (int64_t)p->N + n] : 0.0);", "out[n] = acc;"),
    ("ue8m0_pairs_bytes_swapped", "return (uint8_t)(((uint16_t)word >> (h ? 8 : 0)) & 0xFFu);",
     "return (uint8_t)(((uint16_t)word >> (h ? 0 : 8)) & 0xFFu);"),
    ("ue8m0_pairs_lhs_k_major", "int16_t w = pairs[(g * P + kb / 2) * M + m];",
     "int16_t w = pairs[(g * M + m) * P + kb / 2];"),
    ("ue8m0_pairs_rhs_k_major", "int16_t pw = pairs[(g * P + kb / 2) * Nb + nb];",
     "int16_t pw = pairs[(g * Nb + nb) * P + kb / 2];"),
    ("ue8m0_pairs_rhs_low_byte_only", "ue8m0_pair_half(pw, kb & 1)", "ue8m0_pair_half(pw, 0)"),
    ("bf16_masked_group0", "        const uint16_t *b = p->B + g * (int64_t)p->N * p->K;",
     "        const uint16_t *b = p->B;"),
]


def _pin_calls(o):
    calls = []
    calls.append(lambda: pins.test_e4m3_table_matches_torch_decode(o))
    calls.append(lambda: pins.test_e4m3_table_format_facts(o))
    calls.append(lambda: pins.test_bf16_rne_matches_torch_cast(o))
    for M, N, K in [(3, 129, 384), (129, 3, 128), (5, 128, 384)]:
        calls.append(lambda M=M, N=N, K=K: pins.test_dense_vs_numpy_dequant_matmul(o, M, N, K))
    calls.append(lambda: pins.test_fp8_fp4_vs_numpy_dequant_matmul(o, 17, 130, 640))
    for f in (pins.test_dense_integer_data_exact_vs_int64, pins.test_all_ones_closed_form,
              pins.test_one_hot_rows, pins.test_sign_flip_and_pow2_scaling,
              pins.test_rows_subset_equals_full, pins.test_c_is_added,
              pins.test_contiguous_segments_equal_dense,
              pins.test_contiguous_group_independence_and_permutation,
              pins.test_masked_rows_and_groups, pins.test_masked_negative_and_subset,
              pins.test_ue8m0_points_from_format, pins.test_ue8m0_packing_byte_order_and_layouts,
              pins.test_ue8m0_all_ones_closed_form, pins.test_e2m1_points_from_format,
              pins.test_ue8m0_pairs_worked_example, pins.test_ue8m0_pairs_equal_quads,
              pins.test_ue8m0_pairs_all_ones_closed_form,
              pins.test_fp8_fp4_nibble_order_and_block_scales, pins.test_fp8_fp4_grouped_equal_dense,
              pins.test_k_grouped_equals_dense_nt_on_transposed_operands,
              pins.test_k_grouped_operand_swap_transposes, pins.test_k_grouped_empty_group_and_closed_form):
        calls.append(lambda f=f: f(o))
    calls.append(lambda: pins.test_k_grouped_vs_numpy_dequant_matmul(o, [128, 256, 0, 384], 37, 129))
    calls.append(lambda: pins.test_bf16_decode_matches_torch_for_every_code(o))
    calls.append(lambda: pins.test_bf16_gemm_vs_numpy(o, 37, 129, 200))
    calls.append(lambda: pins.test_bf16_grouped_equal_dense(o))
    calls.append(lambda: pins.test_fp4_fp4_vs_numpy_dequant_matmul(o, 17, 130, 384))
    calls.append(lambda: pins.test_fp4_fp4_operand_swap_and_grouped(o))
    return calls


def test_unmodified_copy_passes_every_pin(tmp_path):
    src = tmp_path / "oracle.c"
    shutil.copy(SRC, src)
    lib = oracle_pkg.build(str(src), str(tmp_path / "liboracle_copy.so"))
    o = Oracle(oracle_pkg.load(lib))
    for call in _pin_calls(o):
        call()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(text.replace(old, new))
    lib = oracle_pkg.build(str(src), str(tmp_path / f"liboracle_{name}.so"))
    o = Oracle(oracle_pkg.load(lib))
    caught = []
    for call in _pin_calls(o):
        try:
            call()
        except (AssertionError, ValueError, IndexError):
            caught.append(call)
    assert caught, f"no pin caught the planted mistake '{name}'"
