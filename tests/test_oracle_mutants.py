"""Plant plausible mistakes in copies of the C oracle (on the CPU) and check the pins catch each.

Every mutant is one textual change to ``oracle/msm_oracle.c`` -- a dropped term, a wrong sign,
an off-by-one index, a swapped adjoint -- compiled with the oracle's own flags into a temporary
directory.  A mutant that passes every pin would mean the pins cannot tell it from the oracle.
"""
import os

import pytest

import oracle
import pins

# (name, original text, replacement, occurrence index to replace (0 = first))
MUTANTS = [
    ("fwd_velocity_reads_h", "v = beta * v + w;", "v = beta * h + w;", 0),
    ("fwd_h_skips_velocity", "h = a * h + v;", "h = a * h + w;", 0),
    ("fwd_exp_sign", "double a = exp(dt * A[d * N + n]);", "double a = exp(-dt * A[d * N + n]);", 0),
    ("fwd_write_drops_delta", "double w = alpha * (g * B[(b * L + t) * N + n] * xt);",
     "double w = alpha * (B[(b * L + t) * N + n] * xt);", 0),
    ("fwd_reads_velocity", "y[(b * L + t) * D + d] += C[(b * L + t) * N + n] * h;",
     "y[(b * L + t) * D + d] += C[(b * L + t) * N + n] * v;", 0),
    ("fwd_skip_uses_delta",
     "y[(b * L + t) * D + d] += Dskip[d] * x[(b * L + t) * D + d];",
     "y[(b * L + t) * D + d] += Dskip[d] * delta[(b * L + t) * D + d];", 0),
    ("fwd_alpha_scales_velocity", "v = beta * v + w;", "v = alpha * beta * v + w;", 0),
    ("plain_write_drops_delta",
     "h = exp(dt * A[d * N + n]) * h + dt * B[(b * L + t) * N + n] * xt;",
     "h = exp(dt * A[d * N + n]) * h + B[(b * L + t) * N + n] * xt;", 0),
    ("bwd_velocity_adjoint_pure_decay", "double gv = gh + beta * gv_next;",
     "double gv = C[j] * dyt + beta * gv_next;", 0),
    ("bwd_exp_path_uses_gv", "ddelta[i] += alpha * B[j] * xt * gv * gd + An * a * hprev * gh;",
     "ddelta[i] += alpha * B[j] * xt * gv * gd + An * a * hprev * gv;", 0),
    ("bwd_dC_off_by_one", "dC[j] += dyt * hs[t + 1];", "dC[j] += dyt * hs[t];", 0),
    ("bwd_hprev_off_by_one", "double hprev = hs[t];", "double hprev = hs[t + 1];", 0),
    ("bwd_dA_drops_a", "dA_rows[(b * D + d) * N + n] += dt * a * hprev * gh",
     "dA_rows[(b * D + d) * N + n] += dt * hprev * gh", 0),
    ("bwd_gh_uses_a_t", "double gh = C[j] * dyt + a_next * gh_next;",
     "double gh = C[j] * dyt + a * gh_next;", 0),
    ("bwd_skip_dx_uses_x", "dx[i] += Dskip[d] * dy[i];", "dx[i] += Dskip[d] * x[i];", 0),
    ("bwd_dB_uses_gh", "dB[j] += alpha * g * xt * gv;", "dB[j] += alpha * g * xt * gh;", 0),
    ("bwd_dx_drops_alpha", "dx[i] += alpha * g * B[j] * gv;", "dx[i] += g * B[j] * gv;", 0),
    ("bwd_dDskip_uses_y", "dD_rows[b * D + d] += dy[i] * x[i];", "dD_rows[b * D + d] += dy[i];", 0),
    # initial state and terminal adjoints
    ("fwd_ignores_v0", "double v = v0 ? v0[(b * D + d) * N + n] : 0.0;", "double v = 0.0;", 0),
    ("bwd_ignores_h0", "hs[0] = h;", "hs[0] = 0.0;", 0),
    ("bwd_terminal_v_scaled", "gv += dlast_v[s_i];", "gv += beta * dlast_v[s_i];", 0),
    ("bwd_drops_terminal_h", "gv_next = 0.0, a_next = 1.0;", "gv_next = 0.0, a_next = 0.0;", 0),
    ("bwd_dh0_drops_a", "dh0[s_i] = L > 0 ? a_next * gh_next", "dh0[s_i] = L > 0 ? gh_next", 0),
    ("bwd_dv0_drops_beta", "dv0[s_i] = L > 0 ? beta * gv_next", "dv0[s_i] = L > 0 ? gv_next", 0),
    # the fused op's extras
    ("fused_softplus_without_bias", "out[i] = delta_softplus ? softplus(u) : u;",
     "out[i] = delta_softplus ? softplus(delta[i]) + (u - delta[i]) : u;", 0),
    ("softplus_drops_linear_part", "return u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u));",
     "return u > 0.0 ? log1p(exp(-u)) : log1p(exp(u));", 0),
    ("fused_gate_is_logistic", "y[i] = z ? yr[i] * silu(z[i]) : yr[i];",
     "y[i] = z ? yr[i] * logistic(z[i]) : yr[i];", 0),
    ("fused_dy_not_gated", "ge[i] = dy[i] * silu(z[i]);", "ge[i] = dy[i];", 0),
    ("fused_dz_logistic_grad", "dz[i] = dy[i] * yr[i] * silu_grad(z[i]);",
     "dz[i] = dy[i] * yr[i] * logistic(z[i]);", 0),
    ("silu_grad_sign", "return s * (1.0 + z * (1.0 - s));", "return s * (1.0 + z * s);", 0),
    ("fused_ddelta_chain_drops_bias",
     "ddelta[i] *= logistic(delta[i] + (delta_bias ? delta_bias[i % D] : 0.0));",
     "ddelta[i] *= logistic(delta[i]);", 0),
    ("fused_dbias_first_row", "for (int64_t b = 0; b < Bt; ++b)\n        for (int64_t t = 0; t < L; ++t)",
     "for (int64_t b = 0; b < 1; ++b)\n        for (int64_t t = 0; t < L; ++t)", 0),
    # zero-order hold
    ("zoh_write_uses_a", "return An == 0.0 ? dt : expm1(dt * An) / An;",
     "return An == 0.0 ? dt : exp(dt * An) / An;", 0),
    ("zoh_ddelta_drops_a", "return zoh ? exp(dt * An) : 1.0;", "return 1.0;", 0),
    ("zoh_dA_drops_g", "return (dt * exp(u) - expm1(u) / An) / An;", "return (dt * exp(u)) / An;", 0),
    ("zoh_ignored_in_fused", "double g = write_coef(dt, A[d * N + n], zoh);",
     "double g = write_coef(dt, A[d * N + n], 0);", 0),
    # complex-valued SSM
    ("complex_adjoint_without_conj", "double complex gh = dyt * conj(Cj) + conj(a_next) * gh_next;",
     "double complex gh = dyt * conj(Cj) + a_next * gh_next;", 0),
    ("complex_readout_conj", "double complex gh = dyt * conj(Cj) + conj(a_next) * gh_next;",
     "double complex gh = dyt * Cj + conj(a_next) * gh_next;", 0),
    ("complex_dA_without_conj", "dAn += conj(dt * a * hprev) * gh;", "dAn += dt * a * hprev * gh;", 0),
    ("complex_dC_without_conj", "double complex gC = dyt * conj(hs[t + 1]);",
     "double complex gC = dyt * hs[t + 1];", 0),
    ("complex_output_imag", "y[(b * L + t) * D + d] += creal(cget(C, (b * L + t) * N + n) * h);",
     "y[(b * L + t) * D + d] += cimag(cget(C, (b * L + t) * N + n) * h);", 0),
]


def _mutate(src, old, new, occ):
    pos = -1
    for _ in range(occ + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, "mutation site not found: %r" % old
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, old, new, occ):
    with open(oracle.SOURCE) as f:
        src = f.read()
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    cpath = os.path.join(str(tmp_path), "mutant_%s.c" % name)
    with open(cpath, "w") as f:
        f.write(mutated)
    so = oracle.compile_source(cpath, os.path.join(str(tmp_path), "libmutant_%s.so" % name))
    orc = oracle.Oracle(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            caught.append((pin.__name__, str(e)[:120]))
    assert caught, "no pin caught mutant %s" % name
