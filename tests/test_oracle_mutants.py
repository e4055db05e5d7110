"""The pins must catch plausible mistakes in the oracle.

Each mutant is a copy of oracle/ssm_oracle.c with one planted error (a dropped
term, a wrong sign, a transposed index, an output lag, ...), compiled with the
same flags into a temporary directory.  Every mutant must fail at least one pin
of tests/pins.py; the real oracle passes them all (test_oracle_pins.py).
"""
import os

import pytest

import oracle
import pins

# (name, original text, replacement)
MUTANTS = [
    ("output_lag", "      h[n] = abar * h[n] + bbar_u;\n      v += C_b[n * seqlen + l] * h[n];",
     "      v += C_b[n * seqlen + l] * h[n];\n      h[n] = abar * h[n] + bbar_u;"),
    ("exp_sign", "exp(delta * A_row[n])", "exp(-delta * A_row[n])"),
    ("dropped_D", "    v += Dd * ul;", "    v += 0.0 * Dd * ul;"),
    ("B_transposed", "delta * B_b[n * seqlen + l] * ul", "delta * B_b[l * dstate + n] * ul"),
    ("C_transposed", "v += C_b[n * seqlen + l] * h[n];", "v += C_b[l * dstate + n] * h[n];"),
    ("bias_ignored", "double x = dt_row[l] + bias;", "double x = dt_row[l] + 0.0 * bias;"),
    ("bias_after_softplus", "double delta = softplus_flag ? oracle_softplus(x) : x;",
     "double delta = softplus_flag ? oracle_softplus(dt_row[l]) + bias : x;"),
    ("gate_sigmoid", "if (z_row) v *= oracle_silu(z_row[l]);", "if (z_row) v *= 1.0 / (1.0 + exp(-z_row[l]));"),
    ("h0_ignored", "h[n] = h0 ? h0[ch * dstate + n] : 0.0;", "h[n] = 0.0;"),
    ("bbar_without_delta", "double bbar_u = delta * B_b[n * seqlen + l] * ul;",
     "double bbar_u = B_b[n * seqlen + l] * ul;"),
    ("softplus_negative_branch", "return (x > 0.0 ? x : 0.0) + log1p(exp(-ax));", "return x + log1p(exp(-ax));"),
    ("A_row_of_channel_0", "delta + ch * seqlen, A + d * dstate,", "delta + ch * seqlen, A,"),
    ("B_of_batch_0", "B + b * dstate * seqlen, C + b * dstate * seqlen,", "B, C + b * dstate * seqlen,"),
    ("abar_linearized", "double abar = exp(delta * A_row[n]);", "double abar = 1.0 + delta * A_row[n];"),
    ("state_not_decayed", "h[n] = abar * h[n] + bbar_u;", "h[n] = h[n] + bbar_u;"),
    ("conv_taps_reversed", "acc += w[d * width + k] * v;", "acc += w[d * width + (width - 1 - k)] * v;"),
    ("conv_off_by_one", "int64_t src = l - (width - 1) + k;", "int64_t src = l - width + k;"),
    ("conv_prev_ignored", "v = x_prev ? x_prev[ch * (width - 1) + (width - 1) + src] : 0.0;", "v = 0.0;"),
    ("conv_prev_reversed", "x_prev[ch * (width - 1) + (width - 1) + src]", "x_prev[ch * (width - 1) - 1 - src]"),
    ("conv_bias_dropped", "double acc = cb ? cb[d] : 0.0;", "double acc = 0.0;"),
    ("conv_silu_dropped", "u[ch * seqlen + l] = silu_flag ? oracle_silu(acc) : acc;", "u[ch * seqlen + l] = acc;"),
    ("bwd_lambda_not_decayed", "          lam[n] *= abar;", "          lam[n] *= 1.0;"),
    ("bwd_hprev_is_h", "const double hprev = hs[t * dstate + n];", "const double hprev = hs[(t + 1) * dstate + n];"),
    ("bwd_softplus_grad_dropped", "softplus_flag ? dstep / (1.0 + exp(-x)) : dstep", "softplus_flag ? dstep : dstep", 0),
    ("bwd_dz_sign", "(1.0 + zt * (1.0 - sg))", "(1.0 - zt * (1.0 - sg))", 0),
    ("bwd_dB_missing_step", "+= lam[n] * phi * ut;", "+= lam[n] * ut;"),
    ("bwd_zoh_dphi_dstep", "const double dphi_dstep = zoh ? abar : 1.0;", "const double dphi_dstep = 1.0;"),
    ("bwd_zoh_dphi_da_dropped", "const double dphi_da = zoh ? oracle_zoh_b_da(step, Ar[n]) : 0.0;",
     "const double dphi_da = 0.0;"),
    ("bwd_zoh_series_term", "term *= x * (double)(k + 2) / ((double)(k + 1) * (double)(k + 3));",
     "term *= x / (double)(k + 3);"),
    ("bwd_zoh_closed_form_sign", "return (delta * exp(x) - expm1(x) / a) / a;", "return (delta * exp(x) + expm1(x) / a) / a;"),
    ("bwd_dC_uses_hprev", "g * hs[(t + 1) * dstate + n];", "g * hs[t * dstate + n];"),
    ("zoh_missing_divide", "expm1(delta * a) / a : delta", "expm1(delta * a) : delta"),
    ("zoh_exp_not_expm1", "expm1(delta * a) / a : delta", "exp(delta * a) / a : delta"),
    ("zoh_zero_limit", "expm1(delta * a) / a : delta", "expm1(delta * a) / a : 0.0"),
    ("zoh_ignored", "      if (zoh) bbar_u = ", "      if (0) bbar_u = "),
    ("zoh_sign", "expm1(delta * a) / a : delta", "expm1(-delta * a) / a : delta"),
    ("zoh_without_B", "oracle_zoh_b(delta, A_row[n]) * B_b[n * seqlen + l] * ul", "oracle_zoh_b(delta, A_row[n]) * ul"),
    ("cplx_no_factor_two", "double v = 2.0 * creal(acc)", "double v = creal(acc)"),
    ("cplx_imag_part_out", "double v = 2.0 * creal(acc)", "double v = 2.0 * cimag(acc)"),
    ("cplx_A_imag_dropped", "cexp(step * (a[0] + I * a[1]))", "cexp(step * (a[0] + 0.0 * I * a[1]))"),
    ("cplx_A_conjugated", "cexp(step * (a[0] + I * a[1]))", "cexp(step * (a[0] - I * a[1]))"),
    ("cplx_B_imag_dropped", "step * (bb[0] + I * bb[1]) * ul", "step * (bb[0] + 0.0 * I * bb[1]) * ul"),
    ("cplx_C_conjugated", "acc += (cc[0] + I * cc[1]) * h[n];", "acc += (cc[0] - I * cc[1]) * h[n];"),
    ("cplx_h0_imag_dropped", "h0[(ch * dstate + n) * 2] + I * h0[(ch * dstate + n) * 2 + 1]",
     "h0[(ch * dstate + n) * 2] + 0.0 * I * h0[(ch * dstate + n) * 2 + 1]", 0),
    ("cplx_bwd_h0_imag_dropped", "h0[(ch * dstate + n) * 2] + I * h0[(ch * dstate + n) * 2 + 1]",
     "h0[(ch * dstate + n) * 2] + 0.0 * I * h0[(ch * dstate + n) * 2 + 1]", 1),
    ("cplx_bwd_adjoint_not_conj", "lam[n] *= conj(abar);", "lam[n] *= abar;"),
    ("cplx_bwd_C_not_conj", "lam[n] += 2.0 * g * conj(cn);", "lam[n] += 2.0 * g * cn;"),
    ("cplx_bwd_dC_factor", "const double complex dc = 2.0 * g * conj(hs[(t + 1) * dstate + n]);",
     "const double complex dc = g * conj(hs[(t + 1) * dstate + n]);"),
    ("cplx_bwd_dA_not_conj", "partA[ch * dstate + n] += lam[n] * conj(step * q);", "partA[ch * dstate + n] += lam[n] * step * q;"),
    ("cplx_bwd_dstep_imag", "dstep += creal(lam[n] * conj(an * q + bn * ut));", "dstep += cimag(lam[n] * conj(an * q + bn * ut));"),
    ("bwd_dD_after_gate", "        partD[ch] += g * ut;", "        partD[ch] += dy[ch * seqlen + t] * ut;", 0),
    # Sites that the real and the complex backward share: the occurrence is named.
    ("cplx_bwd_softplus_grad_dropped", "softplus_flag ? dstep / (1.0 + exp(-x)) : dstep", "softplus_flag ? dstep : dstep", 1),
    ("cplx_bwd_dz_sign", "(1.0 + zt * (1.0 - sg))", "(1.0 - zt * (1.0 - sg))", 1),
    ("cplx_bwd_dD_after_gate", "        partD[ch] += g * ut;", "        partD[ch] += dy[ch * seqlen + t] * ut;", 1),
    ("conv_bwd_silu_grad_dropped", "dv *= s * (1.0 + v * (1.0 - s));", "dv *= s;"),
    ("conv_bwd_silu_at_no_bias", "        double v = cb ? cb[d] : 0.0;\n        double in[4];",
     "        double v = 0.0;\n        double in[4];"),
    ("conv_bwd_dx_taps_reversed", "dx[ch * seqlen + src] += w[d * width + k] * dv;",
     "dx[ch * seqlen + src] += w[d * width + (width - 1 - k)] * dv;"),
    ("conv_bwd_prev_grad_dropped", "dx_prev[ch * hist + hist + src] += w[d * width + k] * dv;",
     "dx_prev[ch * hist + hist + src] += 0.0 * dv;"),
    ("conv_bwd_dw_taps_reversed", "gw[k] += dv * in[k];", "gw[k] += dv * in[width - 1 - k];"),
    ("conv_bwd_bias_grad_dropped", "        gb += dv;", "        gb += 0.0 * dv;"),
]
# A site written twice (the real and the complex backward) is mutated at the
# named occurrence (0 = first); every other site must occur exactly once.
MUTANTS = [m if len(m) == 4 else m + (None,) for m in MUTANTS]


@pytest.fixture(scope="module")
def source():
    return open(oracle.SOURCE).read()


def mutate(source, old, new, nth):
    if nth is None:
        assert source.count(old) == 1, "mutation site not found exactly once: %r" % old
        return source.replace(old, new)
    assert source.count(old) == 2, "shared mutation site not found exactly twice: %r" % old
    at = source.index(old) if nth == 0 else source.index(old, source.index(old) + 1)
    return source[:at] + new + source[at + len(old):]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new, nth):
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(mutate(source, old, new, nth))
    lib = oracle.compile_oracle(str(src), str(tmp_path / ("libmutant_%s.so" % name)))
    o = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
