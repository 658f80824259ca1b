"""The SwiGLU / GeGLU CPU oracle checked against its pins, and planted mistakes in
copies of its C source (built on the CPU) each caught by at least one pin."""
import pytest

from oracle import build as obuild
from oracle import glu as glu_oracle
from glu_oracle_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_glu_oracle_pin(check):
    check(glu_oracle.default())


SRC = open(obuild.GLU_SRC).read()

# (name, text in glu_oracle.c, replacement)
MUTATIONS = [
    ("sigmoid_sign", "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    ("cdf_sign", "0.5 * erfc(-x / sqrt(2.0))", "0.5 * erfc(x / sqrt(2.0))"),
    ("cdf_no_sqrt2", "0.5 * erfc(-x / sqrt(2.0))", "0.5 * erfc(-x)"),
    ("cdf_missing_half", "0.5 * erfc(-x / sqrt(2.0))", "erfc(-x / sqrt(2.0))"),
    ("pdf_unnormalised", "exp(-0.5 * x * x) / sqrt(2.0 * PI)", "exp(-0.5 * x * x)"),
    ("pdf_exponent", "exp(-0.5 * x * x) / sqrt(2.0 * PI)", "exp(-x * x) / sqrt(2.0 * PI)"),
    ("tanh_cubic_coef", "return sqrt(2.0 / PI) * (x + 0.044715 * x * x * x);",
     "return sqrt(2.0 / PI) * (x + 0.04715 * x * x * x);"),
    ("tanh_scale", "return sqrt(2.0 / PI) * (x + 0.044715 * x * x * x);",
     "return sqrt(2.0 * PI) * (x + 0.044715 * x * x * x);"),
    ("tanh_prime_missing_3", "(1.0 + 3.0 * 0.044715 * x * x)", "(1.0 + 0.044715 * x * x)"),
    ("tanh_missing_factor_2", "return e * sigmoid(2.0 * tanh_arg(e));",
     "return e * sigmoid(tanh_arg(e));"),
    ("silu_grad_missing_term", "return s + e * s * sigmoid(-e);", "return s;"),
    ("silu_grad_wrong_sigmoid", "return s + e * s * sigmoid(-e);", "return s + e * s * sigmoid(e);"),
    ("gelu_grad_missing_pdf", "return normal_cdf(e) + e * normal_pdf(e);", "return normal_cdf(e);"),
    ("gelu_grad_sign", "return normal_cdf(e) + e * normal_pdf(e);",
     "return normal_cdf(e) - e * normal_pdf(e);"),
    ("tanh_grad_missing_2", "* 2.0 * tanh_arg_prime(e);", "* tanh_arg_prime(e);"),
    ("tanh_grad_sigmoid_sign", "return s + e * s * sigmoid(-2.0 * u)",
     "return s + e * s * sigmoid(2.0 * u)"),
    ("de_missing_g", "de[r * cols + c] = up * gv * oracle_glu_grad(kind, ev);",
     "de[r * cols + c] = up * oracle_glu_grad(kind, ev);"),
    ("dg_uses_grad", "dg[r * cols + c] = up * oracle_glu_act(kind, ev);",
     "dg[r * cols + c] = up * oracle_glu_grad(kind, ev);"),
    ("fwd_ignores_stride", "int64_t i = r * in_stride + c;\n      h[",
     "int64_t i = r * cols + c;\n      h["),
    ("bwd_dh_with_in_stride", "elem(dtype, dh, r * out_stride + c)",
     "elem(dtype, dh, r * in_stride + c)"),
    ("f16_subnormal_scale", "v = ldexp((double)man, -24);", "v = ldexp((double)man, -25);"),
    ("f16_exponent_bias", "v = ldexp((double)(man + 1024), ex - 25);",
     "v = ldexp((double)(man + 1024), ex - 24);"),
    ("bf16_decode_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("round_ties_away", "double r = nearbyint(x / quantum) * quantum;",
     "double r = round(x / quantum) * quantum;"),
    ("round_truncates", "double r = nearbyint(x / quantum) * quantum;",
     "double r = trunc(x / quantum) * quantum;"),
    ("bf16_precision", "round_to_format(in[i], 8, -126", "round_to_format(in[i], 9, -126"),
    ("f16_min_exponent", "round_to_format(in[i], 11, -14, 65504.0)",
     "round_to_format(in[i], 11, -15, 65504.0)"),
    ("no_overflow_to_inf", "if (fabs(r) > max_finite) return x > 0 ? INFINITY : -INFINITY;", ""),
    ("f16_encode_bias", "uint16_t ex = (uint16_t)(E - 1 + 15);", "uint16_t ex = (uint16_t)(E + 15);"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    assert SRC.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(SRC.replace(old, new))
    lib = obuild.build(str(src), str(tmp_path / f"libmut_{name}.so"))
    o = glu_oracle.GluOracle(lib)
    caught = None
    for check in ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            caught = check.__name__
            break
    assert caught, f"planted mistake {name!r} passed every pin"
