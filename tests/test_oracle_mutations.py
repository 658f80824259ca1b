"""Plants plausible mistakes in copies of the oracle's C source (on the CPU),
builds each copy, and checks that at least one pin fails for every mistake:
evidence that the pins constrain every part of the oracle."""
import os

import pytest

import oracle
from oracle import build as obuild
from oracle_checks import ALL_CHECKS

SRC = open(obuild.SRC).read()

# (name, text in rope_oracle.c, replacement)
MUTATIONS = [
    ("y1_sign", "double y1 = x1 * c - x2 * s;", "double y1 = x1 * c + x2 * s;"),
    ("y2_sign", "double y2 = x2 * c + x1 * s;", "double y2 = x2 * c - x1 * s;"),
    ("transposed_rotation", "double s = (double)dir * (double)sn[j];",
     "double s = -(double)dir * (double)sn[j];"),
    ("backward_not_negated", "double s = (double)dir * (double)sn[j];",
     "double s = (double)sn[j];"),
    ("interleaved_pairing", "double x2 = load_elem(dtype, x, row_off + j + half);",
     "double x2 = load_elem(dtype, x, row_off + (j ^ 1));"),
    ("swapped_halves_store", "y_row[j + half] = (float)y2;", "y_row[j + half] = (float)y1;"),
    ("exponent_missing_2", "long double e = -(2.0L * (long double)j) / (long double)D;",
     "long double e = -((long double)j) / (long double)D;"),
    ("exponent_over_D_minus_2", "long double e = -(2.0L * (long double)j) / (long double)D;",
     "long double e = -(2.0L * (long double)j) / (long double)(D - 2 > 0 ? D - 2 : 1);"),
    ("inv_freq_fp32_pow", "out[j] = (float)powl((long double)theta, e);",
     "out[j] = powf((float)theta, (float)e);"),
    ("angle_in_double", "*c = (float)cosl((long double)angle);",
     "*c = (float)cosl((long double)pos * (long double)inv_freq_j);"),
    ("cos_sin_swapped", "*c = (float)cosl((long double)angle);", "*c = (float)sinl((long double)angle);"),
    ("cos_fp32_libm", "*c = (float)cosl((long double)angle);", "*c = cosf(angle);"),
    ("rotation_in_fp32", "double y1 = x1 * c - x2 * s;",
     "double y1 = (double)((float)x1 * (float)c - (float)x2 * (float)s);"),
    ("positions_not_reset", "int32_t pe = shifted(p, seq_offsets, s);\n      if (pe < 0) continue;\n      float cs",
     "int32_t pe = shifted(t, seq_offsets, s);\n      if (pe < 0) continue;\n      float cs"),
    ("positions_from_1", "if (pos_out) pos_out[t] = pe;", "if (pos_out) pos_out[t] = pe + 1;"),
    ("seqused_ignored", "if (seqused && (int64_t)seqused[s] < len) len = seqused[s];", ""),
    ("row_walk_off_by_one", "if (p >= 0 && p < used_len(cu, seqused, s)) return shifted(p, seq_offsets, s);",
     "if (p >= 0 && p <= used_len(cu, seqused, s)) return shifted(p, seq_offsets, s);"),
    ("offset_sign", "int64_t q = p + (seq_offsets ? (int64_t)seq_offsets[s] : 0);",
     "int64_t q = p - (seq_offsets ? (int64_t)seq_offsets[s] : 0);"),
    ("offset_ignored", "int64_t q = p + (seq_offsets ? (int64_t)seq_offsets[s] : 0);", "int64_t q = p;"),
    ("negative_shift_kept", "return (q < 0 || q > 2147483647LL) ? -1 : (int32_t)q;",
     "return (q < 0) ? (int32_t)(-q) : (int32_t)q;"),
    ("scale_multiplies", "if (scale != 1.0f) p = p / scale;", "if (scale != 1.0f) p = p * scale;"),
    ("scale_ignored", "if (scale != 1.0f) p = p / scale;", ""),
    ("scale_in_double", "float angle = p * inv_freq_j;",
     "float angle = (float)((double)pos / (double)scale * (double)inv_freq_j);"),
    ("ids_off_by_one", "int32_t pe = position_ids[t];", "int32_t pe = position_ids[t] + 1;"),
    ("ids_negative_rotated", "int32_t pe = position_ids[t];\n      if (pe < 0) continue;",
     "int32_t pe = position_ids[t] < 0 ? -position_ids[t] : position_ids[t];\n      if (pe < 0) continue;"),
    ("bf16_ties_not_even", "if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;",
     "if (rest >= 0x8000u) keep += 1u;"),
    ("bf16_truncates", "if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;", ""),
    # binary16 storage decode
    ("f16_exponent_bias_off_by_one", "v = ldexp((double)(man | 0x400), exp - 25);",
     "v = ldexp((double)(man | 0x400), exp - 24);"),
    ("f16_subnormal_scale", "v = ldexp((double)man, -24);", "v = ldexp((double)man, -25);"),
    ("f16_implicit_bit_dropped", "v = ldexp((double)(man | 0x400), exp - 25);",
     "v = ldexp((double)man, exp - 25);"),
    ("f16_inf_nan_swapped", "v = man ? NAN : INFINITY;", "v = man ? INFINITY : NAN;"),
    ("f16_sign_dropped", "return (float)(sign ? -v : v);", "return (float)v;"),
    # caller-supplied cos/sin tables
    ("table_row_not_scaled", "rotate_row(dtype, x, off, y + off, D, cos_tab + (int64_t)pe * half,",
     "rotate_row(dtype, x, off, y + off, D, cos_tab + (int64_t)pe,"),
    ("table_cos_sin_swapped",
     "cos_tab + (int64_t)pe * half,\n                   sin_tab + (int64_t)pe * half, dir);",
     "sin_tab + (int64_t)pe * half,\n                   cos_tab + (int64_t)pe * half, dir);"),
    ("table_last_row_dropped", "if (pe < 0 || pe >= tab_rows)", "if (pe < 0 || pe >= tab_rows - 1)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    assert SRC.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(SRC.replace(old, new))
    lib = obuild.build(str(src), str(tmp_path / f"libmut_{name}.so"))
    o = oracle.Oracle(lib)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            failed.append(check.__name__)
            break
    assert failed, f"planted mistake {name!r} passed every pin"
