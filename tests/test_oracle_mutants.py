"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins in oracle_pins.py catch every one of them."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mx_oracle.c")

# (name, original text, planted mistake).  Swapping the nibble order inside
# decode_elem is not listed: it permutes K within a 32-block identically for
# A and B, which leaves every block dot product, and so C and T, unchanged.
MUTANTS = [
    ("b_pair_swap", "bdec[k] = decode_elem(fmt_b, B + n * rbb, k, t4, t8);",
     "bdec[k] = decode_elem(fmt_b, B + n * rbb, k ^ 1, t4, t8);"),
    ("scale_bias", "pow2[i] = ldexp(1.0, i - 254)", "pow2[i] = ldexp(1.0, i - 253)"),
    ("b_scale_from_a", "unsigned sa = sarow[b], sb = sbrow[b];",
     "unsigned sa = sarow[b], sb = sarow[b];"),
    ("scale_block_index", "unsigned sa = sarow[b], sb = sbrow[b];",
     "unsigned sa = sarow[b], sb = sbrow[nb - 1 - b];"),
    ("dropped_term", "j < 32 * b + 32; ++j)", "j < 32 * b + 31; ++j)"),
    ("e4m3_bias", "ldexp(1.0 + (double)m / 8.0, (int)e - 7)",
     "ldexp(1.0 + (double)m / 8.0, (int)e - 8)"),
    ("e4m3_subnormal", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    ("e4m3_nan", "if (e == 15 && m == 7) return NAN;", ""),
    ("e2m1_subnormal", "0.5 * (double)m : ldexp", "1.0 * (double)m : ldexp"),
    ("e2m1_sign", "    return s ? -mag : mag;\n}\n\n/* E4M3",
     "    return mag;\n}\n\n/* E4M3"),
    ("e2m1_bias", "ldexp(1.0 + 0.5 * (double)m, (int)e - 1)",
     "ldexp(1.0 + 0.5 * (double)m, (int)e)"),
    ("magnitude_not_abs", "q += fabs(prod[j - 32 * b]);", "q += prod[j - 32 * b];"),
    ("group_grid_fine", "double grid = ldexp(1.0, (e - 1) - 12);",
     "double grid = ldexp(1.0, (e - 1) - 20);"),
    ("group_size_16", "for (int gi = 0; gi < 4; ++gi) loss += group_loss(prod + 8 * gi);",
     "for (int gi = 0; gi < 2; ++gi) loss += group_loss(prod + 16 * gi);"),
    ("group_loss_unscaled", "el += loss * w;", "el += loss;"),
    ("scale_nan_ignored", "double w = (sa == 255 || sb == 255) ? NAN : pow2[sa + sb];",
     "double w = pow2[sa + sb];"),
    ("e8m0_bias", "return ldexp(1.0, (int)byte - 127);", "return ldexp(1.0, (int)byte - 128);"),
    ("row_index", "int64_t m = rows ? rows[i0 + i] : i0 + i;\n                    const",
     "int64_t m = rows ? rows[i0] : i0 + i;\n                    const"),
    ("b_row_stride", "bdec[k] = decode_elem(fmt_b, B + n * rbb, k, t4, t8);",
     "bdec[k] = decode_elem(fmt_b, B + n * (rbb - 1), k, t4, t8);"),
    # Mixed formats: an operand decoded with the other operand's format or
    # row pitch.
    ("mixed_a_decoded_as_b", "adec[i * K + k] = decode_elem(fmt_a, A + m * rba, k, t4, t8);",
     "adec[i * K + k] = decode_elem(fmt_b, A + m * rba, k, t4, t8);"),
    ("mixed_b_pitch_of_a", "bdec[k] = decode_elem(fmt_b, B + n * rbb, k, t4, t8);",
     "bdec[k] = decode_elem(fmt_b, B + n * rba, k, t4, t8);"),
    # E5M2.
    ("e5m2_bias", "ldexp(1.0 + (double)m / 4.0, (int)e - 15)", "ldexp(1.0 + (double)m / 4.0, (int)e - 16)"),
    ("e5m2_subnormal", "ldexp((double)m / 4.0, -14)", "ldexp((double)m / 4.0, -15)"),
    ("e5m2_inf_as_nan", "mag = (m == 0) ? INFINITY : NAN;", "mag = NAN;"),
    ("e5m2_double_sums", "if (exact128) block_exact(", "if (0) block_exact("),
    ("e5m2_quant_emax", "emax_of[6] = {0, 2, 8, 15, 2, 4};", "emax_of[6] = {0, 2, 8, 14, 2, 4};"),
    ("e5m2_quant_bias", "bias_of[6] = {0, 1, 7, 15, 1, 3};", "bias_of[6] = {0, 1, 7, 16, 1, 3};"),
    ("e5m2_pair_double_sums", "const int exact128 = fmt_a == MXO_FMT_E5M2 || fmt_b == MXO_FMT_E5M2;",
     "const int exact128 = fmt_a == MXO_FMT_E5M2 && fmt_b == MXO_FMT_E5M2;"),
    # BF16 GEMM.
    ("bf16_decode_shift", "v.u = (uint32_t)(bits & 0xffffu) << 16;", "v.u = (uint32_t)(bits & 0xffffu) << 15;"),
    ("bf16_b_row", "const double *b = bdec + n * K;", "const double *b = bdec + (n / 2) * K;"),
    ("bf16_last_k", "for (int64_t k = 0; k < K; ++k) {\n                c += a[k] * b[k];",
     "for (int64_t k = 0; k < K - 1; ++k) {\n                c += a[k] * b[k];"),
    ("mixed_same_format_entry", "return mxo_gemm_ab(fmt, fmt, M,", "return mxo_gemm_ab(fmt, MXO_FMT_E4M3, M,"),
    # FP6 elements.
    ("e2m3_bias", "ldexp(1.0 + (double)m / 8.0, (int)e - 1);\n    return s ? -mag : mag;\n}\n\n/* FP6 E3M2",
     "ldexp(1.0 + (double)m / 8.0, (int)e - 2);\n    return s ? -mag : mag;\n}\n\n/* FP6 E3M2"),
    ("e3m2_subnormal", "ldexp((double)m / 4.0, -2)", "ldexp((double)m / 4.0, -3)"),
    ("fp6_bit_offset", "const int64_t bit = 6 * k;", "const int64_t bit = 6 * (k ^ 1);"),
    ("fp6_high_byte_dropped", "if ((bit & 7) > 2) v |=", "if ((bit & 7) > 4) v |="),
    # The quantizer.
    ("q_e4m3_emax", "emax_of[6] = {0, 2, 8, 15, 2, 4};", "emax_of[6] = {0, 2, 7, 15, 2, 4};"),
    ("q_e3m2_emax", "emax_of[6] = {0, 2, 8, 15, 2, 4};", "emax_of[6] = {0, 2, 8, 15, 2, 3};"),
    ("q_e2m3_bias", "bias_of[6] = {0, 1, 7, 15, 1, 3};", "bias_of[6] = {0, 1, 7, 15, 2, 3};"),
    ("q_e3m2_max", "maxv_of[6] = {0, 6.0, 448.0, 57344.0, 7.5, 28.0};",
     "maxv_of[6] = {0, 6.0, 448.0, 57344.0, 7.5, 24.0};"),
    ("q_fp6_bit_order", "const int64_t bit = 6 * k + i;", "const int64_t bit = 6 * k + 5 - i;"),
    ("q_ties_away", "nearbyint(a / quantum)", "round(a / quantum)"),
    ("q_no_saturation", "if (a > maxv) a = maxv;", ""),
    ("q_negative_zero", "if (signbit(x[j])) code |= sign_bit;",
     "if (x[j] < 0.0) code |= sign_bit;"),
    ("q_scale_unclamped_low", "s = s < 0 ? 0 : (s > 254 ? 254 : s);",
     "s = s > 254 ? 254 : s;"),
    ("q_log2_off_by_one", "s = (e2 - 1) - emax + 127;", "s = e2 - emax + 127;"),
    ("q_subnormal_grid", "ldexp(1.0, (e < emin ? emin : e) - man)", "ldexp(1.0, e - man)"),
    ("q_nibble_order", "if (k & 1) *byte", "if (!(k & 1)) *byte"),
    ("q_nonfinite_ignored", "if (!isfinite(x[j])) finite = 0;\n                else if",
     "if (0) finite = 0;\n                else if"),
]


def test_mutations_are_distinct_and_apply():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) >= 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src
    mutated = src.replace(old, new)
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-w", str(c), "-o", str(so), "-lm"], check=True)
    mut = oracle.Oracle(str(so))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError):     # a wrong value, or a rejected call
            caught.append(pin.__name__)
    assert caught, "no pin caught mutant %s" % name


# Mistakes planted in the oracle's grouped GEMM (Python): a neighbour's
# weight, an empty group taking a row, row indices not rebased to the group,
# the first group's scales for every group.
GROUPED_MUTANTS = [
    ("weight_of_next_group", "B[g * N:(g + 1) * N]", "B[(g + 1) % G * N:((g + 1) % G + 1) * N]"),
    ("empty_group_takes_a_row", "r0 += m", "r0 += max(m, 1)"),
    ("a_scale_not_rebased", "A_scale[r0:r0 + m]", "A_scale[0:m]"),
    ("b_scale_not_rebased", "B_scale[g * N:(g + 1) * N]", "B_scale[0:N]"),
    ("b_format_dropped", "group_bound=group_bound, fmt_b=fmt_b)", "group_bound=group_bound)"),
]


@pytest.mark.parametrize("name,old,new", GROUPED_MUTANTS, ids=[m[0] for m in GROUPED_MUTANTS])
def test_pins_catch_grouped_mutant(name, old, new):
    import inspect
    import textwrap

    import numpy as np
    src = textwrap.dedent(inspect.getsource(oracle.Oracle.gemm_grouped))
    assert old in src
    ns = {"np": np}
    exec(src.replace(old, new, 1), ns)
    mut = oracle.Oracle()
    mut.gemm_grouped = ns["gemm_grouped"].__get__(mut)
    with pytest.raises((AssertionError, ValueError)):    # a wrong value, or a rejected call
        oracle_pins.pin_grouped(mut)


# The same kind of mistakes in the grouped BF16 GEMM.
GROUPED_BF16_MUTANTS = [
    ("weight_of_next_group", "B[g * N:(g + 1) * N]", "B[(g + 1) % G * N:((g + 1) % G + 1) * N]"),
    ("empty_group_takes_a_row", "r0 += m", "r0 += max(m, 1)"),
    ("rows_not_rebased", "rows=want[pos] - r0", "rows=want[pos]"),
]


@pytest.mark.parametrize("name,old,new", GROUPED_BF16_MUTANTS,
                         ids=[m[0] for m in GROUPED_BF16_MUTANTS])
def test_pins_catch_grouped_bf16_mutant(name, old, new):
    import inspect
    import textwrap

    import numpy as np
    src = textwrap.dedent(inspect.getsource(oracle.Oracle.gemm_grouped_bf16))
    assert old in src
    ns = {"np": np}
    exec(src.replace(old, new, 1), ns)
    mut = oracle.Oracle()
    mut.gemm_grouped_bf16 = ns["gemm_grouped_bf16"].__get__(mut)
    with pytest.raises((AssertionError, ValueError)):
        oracle_pins.pin_grouped_bf16(mut)


# Mistakes planted in the acceptance helpers (oracle/__init__.py): a looser
# bfloat16 ulp, the wrong subnormal spacing or clamp, a doubled tolerance,
# the ulp term added to FP32 output, a loose comparison, NaN or infinities
# accepted whatever the device returned, round-half-up instead of
# round-to-even in the BF16 conversion, and E leaking into the plain count.
HELPER_MUTANTS = [
    ("ulp_one_bit_loose", "ulp = np.ldexp(1.0, expo - 7)", "ulp = np.ldexp(1.0, expo - 6)"),
    ("ulp_clamp", "expo = np.maximum(e - 1, -126)", "expo = np.maximum(e - 1, -127)"),
    ("ulp_zero", "np.ldexp(1.0, -133), ulp)", "np.ldexp(1.0, -132), ulp)"),
    ("ulp_binade", "expo = np.maximum(e - 1, -126)", "expo = np.maximum(e, -126)"),
    ("tolerance_doubled", "b = REL_TOL * np.asarray(T, np.float64)",
     "b = 2 * REL_TOL * np.asarray(T, np.float64)"),
    ("ulp_for_fp32", "    if out_is_bf16:\n        b = b + bf16_ulp(C)",
     "    if True:\n        b = b + bf16_ulp(C)"),
    ("loose_compare", "bad = special_bad | (~special & ~(err <= lim))",
     "bad = special_bad | (~special & (err > 2 * lim))"),
    ("nan_accepts_anything", "np.where(cnan, np.isnan(g), g == ref)",
     "np.where(cnan, True, g == ref)"),
    ("inf_sign_ignored", "np.where(cnan, np.isnan(g), g == ref)",
     "np.where(cnan, np.isnan(g), np.isinf(g))"),
    ("bf16_round_half_up", "rnd = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000",
     "rnd = (bits + 0x8000) & 0xFFFF0000"),
    ("bf16_truncates", "rnd = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000",
     "rnd = bits & 0xFFFF0000"),
    ("plain_count_with_e", "pw, pbad = judge(bound(C, T, out_is_bf16))",
     "pw, pbad = judge(bound(C, T, out_is_bf16, E))"),
    ("zero_limit_lenient", "np.where(err == 0, 0.0, np.inf))", "np.where(err == 0, 0.0, 0.0))"),
]


def _helper_namespace(old=None, new=None):
    import inspect
    import types

    import numpy as np
    src = "\n\n".join(inspect.getsource(f) for f in (oracle.bf16_ulp, oracle.bound,
                                                      oracle.round_to_output, oracle.compare))
    if old is not None:
        assert old in src, old
        src = src.replace(old, new, 1)
    ns = {"np": np, "REL_TOL": oracle.REL_TOL}
    exec(src, ns)
    return types.SimpleNamespace(**{k: ns[k] for k in ("bf16_ulp", "bound", "round_to_output",
                                                        "compare")})


def test_helper_namespace_unmutated_passes():
    h = _helper_namespace()
    for pin in oracle_pins.HELPER_PINS:
        pin(h)


@pytest.mark.parametrize("name,old,new", HELPER_MUTANTS, ids=[m[0] for m in HELPER_MUTANTS])
def test_pins_catch_helper_mutant(name, old, new):
    h = _helper_namespace(old, new)
    caught = []
    for pin in oracle_pins.HELPER_PINS:
        try:
            pin(h)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin caught helper mutant %s" % name
