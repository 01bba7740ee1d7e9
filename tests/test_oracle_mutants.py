"""Planted mistakes in the oracle, on the CPU: every plausible slip (a dropped
term, a wrong sign, a swapped operand or index) must fail at least one pin.
Each mutant is a copy of oracle/kda_oracle.c with one textual change, built
with gcc into a temporary directory."""
import os

import pytest

import oracle_pins as P
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "kda_oracle.c")

MUTANTS = {
    "decay_dropped": ("for (int64_t j = 0; j < dv; ++j) row[j] *= a;",
                      "for (int64_t j = 0; j < dv; ++j) row[j] *= 1.0;"),
    "gate_sign": ("double a = exp((double)J->g[grow + c]);",
                  "double a = exp(-(double)J->g[grow + c]);"),
    "beta_dropped": ("u[j] = b * (", "u[j] = 1.0 * ("),
    "error_sign": ("vrow + j) - acc);", "vrow + j) + acc);"),
    "write_with_q": ("row[j] += kh[c] * u[j];", "row[j] += qh[c] * u[j];"),
    "read_with_k": ("acc += S[c * dv + j] * qh[c];", "acc += S[c * dv + j] * kh[c];"),
    "read_before_write": ("acc += S[c * dv + j] * qh[c];",
                          "acc += (S[c * dv + j] - kh[c] * u[j]) * qh[c];"),
    "transposed_correction": ("acc += S[c * dv + j] * kh[c];", "acc += S[j * dv + c] * kh[c];"),
    "no_l2norm": ("if (J->qk_l2norm) {", "if (0) {"),
    "norm_squared": ("double rq = 1.0 / sqrt(qq + ORACLE_EPS), rk = 1.0 / sqrt(kk + ORACLE_EPS);",
                     "double rq = 1.0 / (qq + ORACLE_EPS), rk = 1.0 / (kk + ORACLE_EPS);"),
    "gate_from_head0": ("(tok * H + h) * dk, tok * H + h,", "(tok * H) * dk, tok * H + h,"),
    "varlen_offset": ("tok0 = J->cu_seqlens[n];", "tok0 = 0 * J->cu_seqlens[n];"),
    "scale_ignored": ("J->o[orow + j] = J->scale * acc;", "J->o[orow + j] = acc;"),
    # output epilogue (head-wise RMSNorm x sigmoid gate)
    "rms_sum_not_mean": ("ms /= (double)dv;", "ms /= 1.0;"),
    "rms_eps_outside": ("1.0 / sqrt(ms + eps);", "1.0 / (sqrt(ms) + eps);"),
    "rms_not_rooted": ("1.0 / sqrt(ms + eps);", "1.0 / (ms + eps);"),
    "gate_swish": ("x * inv_rms * wj * gate;", "x * inv_rms * wj * gate * load_in(z, in_dtype, r * dv + j);"),
    "out_gate_sign": ("exp(-load_in(z, in_dtype, r * dv + j))", "exp(load_in(z, in_dtype, r * dv + j))"),
    "norm_weight_ignored": ("const double wj = w ? (double)w[j] : 1.0;", "const double wj = 1.0;"),
    # ShortConv + Swish
    "conv_taps_reversed": ("acc += (double)w[c * W + i] * ext[t + i];",
                           "acc += (double)w[c * W + (W - 1 - i)] * ext[t + i];"),
    "conv_state_ignored": ("ext[i] = state ? (double)state[(n * C + c) * H + i] : 0.0;",
                           "ext[i] = 0.0;"),
    "conv_state_reversed": ("ext[i] = state ? (double)state[(n * C + c) * H + i] : 0.0;",
                            "ext[i] = state ? (double)state[(n * C + c) * H + (H - 1 - i)] : 0.0;"),
    "conv_no_swish": ("y[(rowbase + t0 + t) * C + c] = acc / (1.0 + exp(-acc));",
                      "y[(rowbase + t0 + t) * C + c] = acc;"),
    "conv_sigmoid_not_swish": ("y[(rowbase + t0 + t) * C + c] = acc / (1.0 + exp(-acc));",
                               "y[(rowbase + t0 + t) * C + c] = 1.0 / (1.0 + exp(-acc));"),
    "conv_bias_ignored": ("double acc = bias ? (double)bias[c] : 0.0;", "double acc = 0.0;"),
    "conv_state_out_first": ("state_out[(n * C + c) * H + i] = ext[len + i];",
                             "state_out[(n * C + c) * H + i] = ext[i];"),
    "conv_varlen_rows": ("ext[H + t] = load_in(x, in_dtype, (rowbase + t0 + t) * C + c);",
                         "ext[H + t] = load_in(x, in_dtype, (rowbase + t) * C + c);"),
    "norm_over_first_row": ("const double x = load_in(o, in_dtype, r * dv + j);\n            ms += x * x;",
                            "const double x = load_in(o, in_dtype, j);\n            ms += x * x;"),
}


def _caught(lib):
    for pin in P.ALL_PINS:
        try:
            pin(lib=lib)
        except (AssertionError, RuntimeError, ValueError):
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    path = tmp_path / f"mut_{name}.c"
    path.write_text(mutated)
    lib = O.open_library(O.compile_source(str(path), str(tmp_path / f"lib_{name}.so")))
    assert _caught(lib) is not None, f"mutant {name} passes every pin"
