"""Plant plausible mistakes in copies of the oracle and check that a pin fails.

Each mutant is a textual edit of ``oracle/oracle_scan.c`` compiled into a
temporary directory (CPU only).  The committed oracle is never modified.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

# (name, [(original text, replacement), ...])
MUTANTS = [
    ("drop_D_term", [("yt += (j->D ? j->D[d] : 0.0) * ut;", "yt += 0.0 * ut;")]),
    ("exp_sign", [("const double abar = exp(dt * j->A[d * N + n]);",
                   "const double abar = exp(-dt * j->A[d * N + n]);")]),
    ("exp_drops_delta", [("const double abar = exp(dt * j->A[d * N + n]);",
                          "const double abar = exp(j->A[d * N + n]);")]),
    ("A_transposed", [("const double abar = exp(dt * j->A[d * N + n]);",
                       "const double abar = exp(dt * j->A[n * Dn + d]);")]),
    ("bbar_drops_delta", [("        return dt * b;\n", "        return b;\n")]),
    ("B_C_swapped", [("oracle_bbar(dt, j->A[d * N + n], j->B[bln + n], j->zoh)",
                      "oracle_bbar(dt, j->A[d * N + n], j->C[bln + n], j->zoh)"),
                     ("yt += j->C[bln + n] * h[n];", "yt += j->B[bln + n] * h[n];")]),
    ("zoh_drops_inverse_A", [("return expm1(dt * a) / a * b;", "return expm1(dt * a) * b;")]),
    ("zoh_exp_not_expm1", [("return expm1(dt * a) / a * b;", "return exp(dt * a) / a * b;")]),
    ("zoh_ignored", [("    if (!zoh || a == 0.0)", "    if (1)")]),
    ("zoh_extra_delta", [("return expm1(dt * a) / a * b;", "return dt * expm1(dt * a) / a * b;")]),
    ("C_previous_step", [("yt += j->C[bln + n] * h[n];",
                          "yt += j->C[(bln >= N ? bln - N : bln) + n] * h[n];")]),
    ("readout_before_update", [
        ("            /* discretise and advance the state */\n",
         "            double ypre = 0.0;\n"
         "            for (int64_t n = 0; n < N; ++n) ypre += j->C[bln + n] * h[n];\n"),
        ("            double yt = 0.0;\n            for (int64_t n = 0; n < N; ++n)\n"
         "                yt += j->C[bln + n] * h[n];\n",
         "            double yt = ypre;\n")]),
    ("no_softplus", [("const double dt = oracle_softplus(j->delta[bld] + (j->bias ? j->bias[d] : 0.0));",
                      "const double dt = j->delta[bld] + (j->bias ? j->bias[d] : 0.0);")]),
    ("bias_outside_softplus", [
        ("const double dt = oracle_softplus(j->delta[bld] + (j->bias ? j->bias[d] : 0.0));",
         "const double dt = oracle_softplus(j->delta[bld]) + (j->bias ? j->bias[d] : 0.0);")]),
    ("softplus_drops_x", [("return x + log1p(exp(-x));", "return log1p(exp(-x));")]),
    ("silu_sign", [("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));")]),
    ("gate_is_sigmoid", [("yt *= oracle_silu(j->z[bld]);",
                          "yt *= 1.0 / (1.0 + exp(-j->z[bld]));")]),
    ("h0_ignored", [("h[n] = j->h0 ? j->h0[(b * Dn + d) * N + n] : 0.0;", "h[n] = 0.0;")]),
    ("h_last_wrong_index", [("j->h_last[(b * Dn + d) * N + n] = h[n];",
                             "j->h_last[(b * Dn + d) * N + n] = h[0];")]),
    ("u_from_wrong_channel", [("const double ut = j->u[bld];",
                               "const double ut = j->u[bld - d];")]),
    ("step_drops_delta_in_bbar", [("oracle_bbar(dt, A[d * d_state + n], B[b * d_state + n], zoh)",
                                   "B[b * d_state + n]")]),
    ("step_no_gate", [("            if (z)\n                yt *= oracle_silu(z[bd]);\n", "")]),
    # gradients
    ("bwd_mu_no_decay", [("mu[n] *= abar;                               /* Abar_t mu_t",
                          "mu[n] *= 1.0;                                /* Abar_t mu_t")]),
    ("bwd_dB_no_dt", [("j->dB[bln + n] += mu[n] * dt * ut;", "j->dB[bln + n] += mu[n] * ut;")]),
    ("bwd_dC_old_state", [("j->dC[bln + n] += ds * hs[(t + 1) * N + n];",
                           "j->dC[bln + n] += ds * hs[t * N + n];")]),
    ("bwd_dA_no_abar", [("j->dA_part[(b * Dn + d) * N + n] += mu[n] * dt * abar * hprev;",
                         "j->dA_part[(b * Dn + d) * N + n] += mu[n] * dt * hprev;")]),
    ("bwd_softplus_grad_sign", [("const double dv = ddt / (1.0 + exp(-v));",
                                 "const double dv = ddt / (1.0 + exp(v));")]),
    ("bwd_dz_no_dgate", [("j->dz[bld] = j->z ? j->dy[bld] * s * dgate : 0.0;",
                          "j->dz[bld] = j->z ? j->dy[bld] * s : 0.0;")]),
    ("bwd_du_no_D", [("double ddt = 0.0, du = ds * (j->D ? j->D[d] : 0.0);",
                      "double ddt = 0.0, du = 0.0;")]),
    ("bwd_ddt_no_input_term", [("ddt += mu[n] * (a * abar * hprev + j->B[bln + n] * ut);",
                                "ddt += mu[n] * (a * abar * hprev);")]),
    # exponential-trapezoidal rule
    ("trap_weights_swapped", [("return (1.0 - lam) * dt * b_prev * u_prev + lam * dt * b * u;",
                               "return lam * dt * b_prev * u_prev + (1.0 - lam) * dt * b * u;")]),
    ("trap_lookback_not_advanced", [("            u_lb = ut;\n", "")]),
    ("trap_lookback_current_B", [("B_lb ? B_lb[n] : 0.0, u_lb)", "j->B[bln + n], u_lb)")]),
    ("trap_lookback_decayed", [("return (1.0 - lam) * dt * b_prev * u_prev + lam * dt * b * u;",
                                "return (1.0 - lam) * dt * b_prev * u_prev * exp(-dt) + "
                                "lam * dt * b * u;")]),
    ("trap_u_prev_ignored", [("double u_lb = j->u_prev ? j->u_prev[b * Dn + d] : 0.0;",
                              "double u_lb = 0.0;")]),
    ("trap_step_no_u_prev", [("u_prev ? u_prev[bd] : 0.0)", "0.0)")]),
    # data-dependent rotation
    ("rot_transposed", [("h[2 * k] = c * x - s * w;", "h[2 * k] = c * x + s * w;"),
                        ("h[2 * k + 1] = s * x + c * w;", "h[2 * k + 1] = -s * x + c * w;")]),
    ("rot_angle_without_delta", [("const double phi = dt * theta[k];",
                                  "const double phi = theta[k];")]),
    ("rot_previous_step_angle", [("oracle_rotate(h, j->theta + (b * j->L + t) * (N / 2), dt, N);",
                                  "oracle_rotate(h, j->theta + (b * j->L + (t > 0 ? t - 1 : 0)) "
                                  "* (N / 2), dt, N);")]),
    ("rot_pairs_adjacent_halves", [("const double x = h[2 * k], w = h[2 * k + 1];",
                                    "const double x = h[k], w = h[k + N / 2];")]),
    ("rot_step_missing", [("                oracle_rotate(hb, theta + b * (d_state / 2), dt, d_state);\n",
                           "")]),
    # gradients of the zero-order hold, the trapezoid and the rotation
    ("bwdx_zoh_dA_term_dropped", [("dAn += mu[n] * Bn * ut * (a != 0.0 ? (dt * abar - beta) / a",
                                   "dAn += 0.0 * mu[n] * Bn * ut * (a != 0.0 ? (dt * abar - beta) / a")]),
    ("bwdx_zoh_ddt_no_abar", [("ddt += mu[n] * Bn * ut * abar;", "ddt += mu[n] * Bn * ut;")]),
    ("bwdx_zoh_du_euler", [("du += mu[n] * beta * Bn;", "du += mu[n] * dt * Bn;")]),
    ("bwdx_zoh_limit_wrong", [(": 0.5 * dt * dt);", ": dt * dt);")]),
    ("bwdx_trap_lookback_not_carried", [("lbk[n] = mu[n] * (1.0 - lam) * dt;", "lbk[n] = 0.0;")]),
    ("bwdx_trap_lookback_lambda", [("lbk[n] = mu[n] * (1.0 - lam) * dt;",
                                    "lbk[n] = mu[n] * lam * dt;")]),
    ("bwdx_trap_dlam_sign", [("dl += mu[n] * dt * (Bn * ut - bp * up);",
                              "dl += mu[n] * dt * (bp * up - Bn * ut);")]),
    ("bwdx_trap_du_prev_ignored", [("dup += lbk[n] * bp;", "dup += 0.0 * bp;")]),
    ("bwdx_rot_not_transposed", [("mu[2 * k] = c * nu[2 * k] + sn * nu[2 * k + 1];",
                                  "mu[2 * k] = c * nu[2 * k] - sn * nu[2 * k + 1];"),
                                 ("mu[2 * k + 1] = -sn * nu[2 * k] + c * nu[2 * k + 1];",
                                  "mu[2 * k + 1] = sn * nu[2 * k] + c * nu[2 * k + 1];")]),
    ("bwdx_rot_dphi_sign", [("const double dphi = nu[2 * k + 1] * hp[0] - nu[2 * k] * hp[1];",
                             "const double dphi = nu[2 * k] * hp[1] - nu[2 * k + 1] * hp[0];")]),
    ("bwdx_rot_dtheta_no_dt", [("j->dtheta[(b * L + t) * K + k] += dt * dphi;",
                                "j->dtheta[(b * L + t) * K + k] += dphi;")]),
    ("bwdx_rot_state_unrotated", [("oracle_rotate(hp, j->theta + (b * L + t) * K, dt, N);",
                                   "(void)hp;")]),
]


def _build_mutant(tmp_path, name, edits):
    with open(oracle.SOURCE) as f:
        src = f.read()
    for old, new in edits:
        assert src.count(old) >= 1, f"{name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    cpath = os.path.join(tmp_path, f"{name}.c")
    with open(cpath, "w") as f:
        f.write(src)
    return oracle.Oracle(oracle.build(cpath, os.path.join(tmp_path, f"lib{name}.so")))


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, edits):
    orc = _build_mutant(str(tmp_path), name, edits)
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except (ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
