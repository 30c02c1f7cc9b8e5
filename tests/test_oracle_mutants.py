"""The oracle pins must notice a planted mistake.

Each case copies ``oracle/oracle.c``, plants one plausible mistake in the copy
(a wrong sign, a dropped term, a transposed index ...), builds it on the CPU
and runs the pin suite against it in a subprocess: the suite has to fail.
Nothing here touches the GPU or the HIP library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "exp_sign": ("double dA = exp(dt * Arow[n]);", "double dA = exp(-dt * Arow[n]);"),
    "no_softplus": ("double dt = softplus ? sp64(xv) : xv;", "double dt = xv;"),
    "bias_index": ("drow[t] + (bias ? bias[d] : 0.0)", "drow[t] + (bias ? bias[0] : 0.0)"),
    "input_no_delta": ("h[n] = dA * h[n] + dt * Bb[n * nl + t] * ut;", "h[n] = dA * h[n] + Bb[n * nl + t] * ut;"),
    "c_transposed": ("acc += Cb[n * nl + t] * h[n];", "acc += Cb[t * nn + n] * h[n];"),
    "b_transposed": ("h[n] = dA * h[n] + dt * Bb[n * nl + t] * ut;", "h[n] = dA * h[n] + dt * Bb[t * nn + n] * ut;"),
    "a_transposed": ("double dA = exp(dt * Arow[n]);", "double dA = exp(dt * A[n * nd + d]);"),
    "skip_outside_gate": ("double yv = acc + (Dv ? Dv[d] * ut : 0.0);\n                if (zrow) yv *= silu64(zrow[t]);",
                          "double yv = acc;\n                if (zrow) yv *= silu64(zrow[t]);\n                yv += (Dv ? Dv[d] * ut : 0.0);"),
    "last_transposed": ("last[row * nn + n] = h[n];", "last[n * rows + row] = h[n];"),
    "h0_ignored": ("h[n] = h0 ? h0[row * nn + n] : 0.0;", "h[n] = 0.0;"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "m2_group": ("const int64_t g = hh / heads_per_group;", "const int64_t g = hh % ng;"),
    "m2_dt_head": ("double xv = dt[bt * nh + hh] + (dtb ? dtb[hh] : 0.0);", "double xv = dt[bt * nh + (hh % 1)] + (dtb ? dtb[hh] : 0.0);"),
    "m2_state_order": ("s[n] = dA * s[n] + delt * Bt[n] * xt;", "s[n] = dA * s[n] + delt * Bt[nn - 1 - n] * xt;"),
    "m2_h0_ignored": ("s[n] = h0 ? h0[unit * nn + n] : 0.0;", "s[n] = 0.0;"),
    "m2_h0_transposed": ("s[n] = h0 ? h0[unit * nn + n] : 0.0;",
                         "s[n] = h0 ? h0[((b * nh + hh) * nn + n) * np + p] : 0.0;"),
    "bwd_adjoint_undecayed": ("lam[n] = a * l;", "lam[n] = l;"),
    "bwd_no_state_path": ("ddl += l * (bb * ur[t] + A[d * nn + n] * a * hp);", "ddl += l * (bb * ur[t]);"),
    "bwd_softplus_derivative": ("ddl / (1.0 + exp(-x))", "ddl / (1.0 + exp(x))"),
    "bwd_dc_previous_state": ("dCm[(b * nn + n) * nl + t] += dy * h[(t + 1) * nn + n];",
                              "dCm[(b * nn + n) * nl + t] += dy * h[t * nn + n];"),
    "bwd_h0_ignored": ("/* forward, keeping every state */\n            for (int64_t n = 0; n < nn; ++n) h[n] = h0 ? h0[row * nn + n] : 0.0;",
                       "/* forward, keeping every state */\n            for (int64_t n = 0; n < nn; ++n) h[n] = 0.0;"),
    "m2_bwd_db_one_head": ("dBt[n] += l * dl[t] * xt;", "if (hh % hpg == 0) dBt[n] += l * dl[t] * xt;"),
    "m2_bwd_ddt_last_channel": ("ddt[(b * nl + t) * nh + hh] += dv;", "ddt[(b * nl + t) * nh + hh] = dv;"),
    "m2_bwd_adjoint_undecayed": ("lam[n] = a * l;   /* a_t lam_t, carried to token t-1 */\n                    }\n                    dx[e] = dxt;",
                                 "lam[n] = l;   /* a_t lam_t, carried to token t-1 */\n                    }\n                    dx[e] = dxt;"),
    "m2_bwd_da_no_delta": ("dA[hh] += l * dl[t] * a * hp;", "dA[hh] += l * a * hp;"),
    "conv_kernel_reversed": ("if (s >= 0) acc += w[d * nk + k] * xr[s];", "if (s >= 0) acc += w[d * nk + (nk - 1 - k)] * xr[s];"),
    "conv_offset": ("const int64_t s = t - (nk - 1) + k;", "const int64_t s = t - nk + k;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new, 1))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(mutant), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, SELSCAN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not notice mutant {name}:\n{r.stdout[-2000:]}"
