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
    # backward (reverse sweep)
    "bwd_readout_old_state": ("for (int64_t j = 0; j < dv; ++j) acc += Sn[c * dv + j] * don[j];",
                              "for (int64_t j = 0; j < dv; ++j) acc += Sp[c * dv + j] * don[j];"),
    "bwd_readout_scale": ("dqh[c] = J->scale * acc;", "dqh[c] = acc;"),
    "bwd_state_from_q_dropped": ("dS[c * dv + j] += J->scale * qh_c * don[j];",
                                 "dS[c * dv + j] += 0.0 * qh_c * don[j];"),
    "bwd_dk_write_dropped": ("acc += dS[c * dv + j] * (b * e[j]);",
                             "acc += 0.0 * dS[c * dv + j] * (b * e[j]);"),
    "bwd_dbeta_uses_u": ("db += du[j] * e[j];", "db += du[j] * b * e[j];"),
    "bwd_dv_no_beta": ("J->grad_v[row_v + j] = b * du[j];", "J->grad_v[row_v + j] = du[j];"),
    "bwd_correction_sign": ("dS[c * dv + j] -= kh_c * (b * du[j]);",
                            "dS[c * dv + j] += kh_c * (b * du[j]);"),
    "bwd_dk_correction_dropped": ("dkh[c] -= acc;", "dkh[c] -= 0.0 * acc;"),
    "bwd_dg_prev_state": ("acc += dS[c * dv + j] * St[c * dv + j];",
                          "acc += dS[c * dv + j] * Sp[c * dv + j];"),
    "bwd_no_decay_back": ("for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] *= a;",
                          "for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] *= 1.0;"),
    "bwd_norm_no_projection": ("J->grad_k[row_k + c] = rk * dkh[c] - rk * rk * rk * kd * kx[c];",
                               "J->grad_k[row_k + c] = rk * dkh[c];"),
    "bwd_norm_q_with_k": ("J->grad_q[row_k + c] = rq * dqh[c] - rq * rq * rq * qd * qx[c];",
                          "J->grad_q[row_k + c] = rq * dqh[c] - rq * rq * rq * qd * kx[c];"),
    "bwd_dfinal_ignored": ("dS[i] = J->dfinal ? (double)J->dfinal[sidx + i] : 0.0;",
                           "dS[i] = 0.0;"),
    "bwd_block_restart": ("memcpy(blk, kept + b * sz, (size_t)sz * sizeof(double));",
                          "memcpy(blk, kept, (size_t)sz * sizeof(double));"),
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
