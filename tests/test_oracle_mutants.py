"""Plant plausible mistakes in copies of the oracle and check that the pins
in tests/test_oracle_pins.py catch every one of them.

Each mutant is a one-line edit of oracle/oracle.c (a dropped term, a flipped
sign, a wrong index or divisor, a swapped operand), compiled on the CPU into a
temporary library; the pin suite of the function it breaks (RMSNorm or
LayerNorm) is run against it in a child process and must fail. The oracle
source in the repository is never modified.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "eps_dropped": ("sumsq / (double)N + eps", "sumsq / (double)N"),
    "rstd_not_inverted": ("r = 1.0 / sqrt(sumsq", "r = sqrt(sumsq"),
    "forward_gamma_dropped": ("y[row * N + j] = up(a, dtype, row * N + j) * r * up(gamma, dtype, j);",
                              "y[row * N + j] = up(a, dtype, row * N + j) * r;"),
    "c1_divisor_n_minus_1": ("\n    c1 /= (double)N;", "\n    c1 /= (double)(N > 1 ? N - 1 : 1);"),
    "c1_not_divided": ("\n    c1 /= (double)N;", "\n"),
    "dx_sign_flipped": ("dx_row[j] = (wdy - x_hat * c1) * r;", "dx_row[j] = (wdy + x_hat * c1) * r;"),
    "dx_c1_term_dropped": ("dx_row[j] = (wdy - x_hat * c1) * r;", "dx_row[j] = wdy * r;"),
    "dx_final_rstd_dropped": ("dx_row[j] = (wdy - x_hat * c1) * r;", "dx_row[j] = wdy - x_hat * c1;"),
    "dgamma_uses_wdy": ("dgamma[j] += dyj * x_hat;\n    }", "dgamma[j] += wdy * x_hat;\n    }"),
    "dgamma_uses_x": ("dgamma[j] += dyj * x_hat;\n    }", "dgamma[j] += dyj * up(x, dtype, row * N + j);\n    }"),
    "gamma_wrong_index": ("double wdy = up(dy, dtype, row * N + j) * up(gamma, dtype, j);",
                          "double wdy = up(dy, dtype, row * N + j) * up(gamma, dtype, (j + row) % N);"),
    "x_hat_reads_dy": ("double x_hat = up(x, dtype, row * N + j) * r;\n        double wdy",
                       "double x_hat = up(dy, dtype, row * N + j) * r;\n        double wdy"),
    "c1_misses_rstd": ("double x_hat = up(x, dtype, row * N + j) * r;\n        double wdy",
                       "double x_hat = up(x, dtype, row * N + j);\n        double wdy"),
    "fused_dres_subtracted": ("d_added[j] += up(dresidual_out", "d_added[j] -= up(dresidual_out"),
    "fused_sum_is_difference": ("(float)up(x, dtype, k) + (float)up(residual", "(float)up(x, dtype, k) - (float)up(residual"),
    "encode_ties_away": ("q = (uint64_t)nearbyint(", "q = (uint64_t)round("),
    "decode_subnormal_scale": ("ldexp((double)m, 1 - bias - f.mbits)", "ldexp((double)m, -bias - f.mbits)"),
    "decode_bias_off_by_one": ("(int)e - bias - f.mbits)", "(int)e - bias - f.mbits + 1)"),
    "bf16_widen_shift": ("uint32_t w = (uint32_t)bits << 16;", "uint32_t w = (uint32_t)bits << 15;"),
    "fused_dres_dropped": ("d_added[j] += up(dresidual_out", "d_added[j] += 0.0 * up(dresidual_out"),
    "rstd_stored_as_sqrt_ms": ("rstd[row] = (float)r;", "rstd[row] = (float)(1.0 / r);"),
}

# LayerNorm mutants, caught by tests/test_oracle_ln_pins.py
LN_MUTANTS = {
    "ln_var_divisor_n_minus_1": ("var /= (double)N;", "var /= (double)(N > 1 ? N - 1 : 1);"),
    "ln_var_without_mean": ("double d = up(x, dtype, i * N + j) - mu;", "double d = up(x, dtype, i * N + j);"),
    "ln_eps_outside_sqrt": ("r = 1.0 / sqrt(var + eps);", "r = 1.0 / (sqrt(var) + eps);"),
    "ln_mean_not_divided": ("mu /= (double)N;", ""),
    "ln_beta_dropped": ("y[i * N + j] = beta ? v + up(beta, dtype, j) : v;", "y[i * N + j] = v;"),
    "ln_forward_gamma_dropped": ("double v = (up(x, dtype, i * N + j) - mu) * r * up(gamma, dtype, j);",
                                 "double v = (up(x, dtype, i * N + j) - mu) * r;"),
    "ln_mean_saved_unscaled": ("mean[i] = (float)mu;", "mean[i] = (float)(mu * (double)N);"),
    "ln_c2_dropped": ("dx[i * N + j] = (wdy - x_hat * c1 - c2) * r;", "dx[i * N + j] = (wdy - x_hat * c1) * r;"),
    "ln_c2_sign_flipped": ("dx[i * N + j] = (wdy - x_hat * c1 - c2) * r;", "dx[i * N + j] = (wdy - x_hat * c1 + c2) * r;"),
    "ln_c1_sign_flipped": ("dx[i * N + j] = (wdy - x_hat * c1 - c2) * r;", "dx[i * N + j] = (wdy + x_hat * c1 - c2) * r;"),
    "ln_c2_not_divided": ("c2 /= (double)N;", ""),
    "ln_c1_not_divided": ("c1 /= (double)N;\n        c2 /= (double)N;", "c2 /= (double)N;"),
    "ln_dx_rstd_dropped": ("dx[i * N + j] = (wdy - x_hat * c1 - c2) * r;", "dx[i * N + j] = wdy - x_hat * c1 - c2;"),
    "ln_bwd_x_hat_without_mean": ("double x_hat = (up(x, dtype, i * N + j) - mu) * r;\n            double wdy = up(dy",
                                  "double x_hat = up(x, dtype, i * N + j) * r;\n            double wdy = up(dy"),
    "ln_c2_misses_gamma": ("double wdy = up(dy, dtype, i * N + j) * up(gamma, dtype, j);\n            c1 += x_hat * wdy;\n            c2 += wdy;",
                           "double wdy = up(dy, dtype, i * N + j) * up(gamma, dtype, j);\n            c1 += x_hat * wdy;\n            c2 += up(dy, dtype, i * N + j);"),
    "ln_dgamma_uses_wdy": ("dgamma[j] += dyj * x_hat;\n            if (dbeta)", "dgamma[j] += wdy * x_hat;\n            if (dbeta)"),
    "ln_dbeta_uses_wdy": ("dbeta[j] += dyj;", "dbeta[j] += wdy;"),
    "ln_gamma_wrong_index": ("double wdy = up(dy, dtype, i * N + j) * up(gamma, dtype, j);\n            c1 +=",
                             "double wdy = up(dy, dtype, i * N + j) * up(gamma, dtype, (j + 1) % N);\n            c1 +="),
}

PINS = {name: "test_oracle_pins.py" for name in MUTANTS}
PINS.update({name: "test_oracle_ln_pins.py" for name in LN_MUTANTS})
MUTANTS.update(LN_MUTANTS)


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    msrc = tmp_path / "oracle_mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mutant.so")
    obuild.build(out=lib, src=str(msrc), extra_flags=["-Wno-error"])
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", PINS[name])],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
