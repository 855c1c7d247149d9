"""Planted mistakes: each plausible slip in the oracle must trip at least one pin.

Every mutant is a copy of oracle/fp4_oracle.c with one textual change, compiled into a
temporary directory and routed in with ``oracle.using``.  The product path is not
involved.  A mutant that every pin accepts means the pins cannot see that class of
mistake, and the test fails.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "tie_to_odd": ("(d == best_d && (i & 1) == 0)", "(d == best_d && (i & 1) == 1)"),
    "no_saturation": ("if (u > 6.0) u = 6.0;", ";"),
    "inverted_multiplier": ("*r = 6.0f / amax;", "*r = amax / 6.0f;"),
    "inverted_dequant_scale": ("*s = amax / 6.0f;", "*s = 6.0f / amax;"),
    "range_without_shift": ("*r = 6.0f / amax;", "*r = 1.0f / amax;"),
    "nibbles_swapped": ("(uint8_t)(orc_e2m1_encode(y0) | (orc_e2m1_encode(y1) << 4));",
                        "(uint8_t)((orc_e2m1_encode(y0) << 4) | orc_e2m1_encode(y1));"),
    "row_max_without_abs": ("float v = fabsf(x[j]);", "float v = x[j];"),
    "quantile_higher": ("return (int64_t)floor(q * (double)(n - 1));",
                        "return (int64_t)ceil(q * (double)(n - 1));"),
    "outlier_ge": ("if (fabsf(a) > T) {", "if (fabsf(a) >= T) {"),
    "clamp_loses_sign": ("ac = copysignf(T, a);", "ac = T;"),
    "delta_sign": ("coo_val[nnz] = a - ac;", "coo_val[nnz] = ac - a;"),
    "bf16_widen": ("uint32_t b = (uint32_t)((const uint16_t *)X)[i] << 16;",
                   "uint32_t b = (uint32_t)((const uint16_t *)X)[i] << 15;"),
    "w_nibble_parity": ("twice_value(w[k / 2], k)", "twice_value(w[k / 2], k + 1)"),
    "decode_table_typo": ("{0, 1, 2, 3, 4, 6, 8, 12}", "{0, 1, 2, 3, 4, 5, 8, 12}"),
    "epilogue_row_scale_twice": ("return t * sw;", "return t * sa;"),
    "epilogue_drops_row_scale": ("float t = acc * sa;", "float t = acc;"),
    "compensation_transposed_w": ("(int64_t)coo_col[e] * N + n", "(int64_t)n * N + coo_col[e]"),
    "compensation_dropped": ("d += t;", "d += 0.0 * t;"),
    "e4m3_bias_8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    "expand_nibbles_swapped": ("out[2 * i] = (uint8_t)orc_e2m1_to_e4m3(packed[i] & 15);",
                               "out[2 * i] = (uint8_t)orc_e2m1_to_e4m3(packed[i] >> 4);"),
    "e4m3_tie_to_odd": ("if (d < best_d || (d == best_d && (b & 1) == 0)) {",
                        "if (d < best_d || (d == best_d && (b & 1) == 1)) {"),
    "e4m3_drops_largest_code": ("for (int b = 1; b < 0x7F; ++b) {  /* the finite positive codes",
                                "for (int b = 1; b < 0x7E; ++b) {  /* the finite positive codes"),
    "fp8_scale_inverted": ("s = amax / 448.0f;", "s = 448.0f / amax;"),
    "col_scale_per_tensor": ("for (int64_t n = 0; n < N; ++n) vector_scale(amax[n], &r[n], &scales[n]);",
                             "for (int64_t n = 1; n < N; ++n) if (amax[n] > amax[0]) amax[0] = amax[n];\n"
                             "    for (int64_t n = 0; n < N; ++n) vector_scale(amax[0], &r[n], &scales[n]);"),
    "transpose_nibble_parity": ("out[c * (R / 2) + r / 2] |= (uint8_t)(code << (4 * (r & 1)));",
                                "out[c * (R / 2) + r / 2] |= (uint8_t)(code << (4 * (c & 1)));"),
    "bwd_row_mult_dropped": ("G[i * C + j] = load_elem(X, dtype, i * C + j) * col_mult[j];",
                             "G[i * C + j] = load_elem(X, dtype, i * C + j);"),
    "bwd_col_mult_dropped": ("H[i * C + j] = row_mult[i] * load_elem(X, dtype, i * C + j);",
                             "H[i * C + j] = load_elem(X, dtype, i * C + j);"),
    "bwd_dA_scale_of_row0": ("dA[m * K + k] = scale_one(dA[m * K + k], sG[m]);",
                             "dA[m * K + k] = scale_one(dA[m * K + k], sG[0]);"),
    "bwd_dW_scale_of_col0": ("dW[k * N + n] = scale_one(dW[k * N + n], sH[n]);",
                             "dW[k * N + n] = scale_one(dW[k * N + n], sH[0]);"),
    "output_pairs_scale_index": ("float ym = dequant_one(acc[i], sA[ms[i]], sW[ns[i]]);",
                                 "float ym = dequant_one(acc[i], sA[ns[i]], sW[ns[i]]);"),
    "output_pairs_entries_of_other_row": ("Y[i] = compensate_one(ym, ms[i], ns[i], N,",
                                          "Y[i] = compensate_one(ym, ns[i], ns[i], N,"),
    "denom_inflated": ("s += fabs(t);", "s += 2.0 * fabs(t);"),
    "denom_without_ymain": ("double d = 0.0, s = fabs((double)ymain);", "double d = 0.0, s = 0.0;"),
    "bwd_scale_pairs_index": ("out[i] = scale_one(acc[i], s[idx[i]]);", "out[i] = scale_one(acc[i], s[i % 1]);"),
}


def _first_failing_pin():
    for pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            return pin.__name__
        except Exception as e:  # an exception is a detection too (e.g. capacity exceeded)
            return f"{pin.__name__} ({type(e).__name__})"
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not unique in the oracle"
    path = tmp_path / "fp4_oracle_mutant.c"
    path.write_text(src.replace(before, after))
    lib = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(src=str(path), out=lib)
    with oracle.using(lib):
        caught = _first_failing_pin()
    assert caught is not None, f"no pin detects the planted mistake {name!r}"


def test_unmutated_oracle_passes_all_pins():
    assert os.path.exists(oracle.load()._name)
    assert _first_failing_pin() is None
