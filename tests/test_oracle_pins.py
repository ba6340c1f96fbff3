"""CPU tests: the oracle against its pins, and the pins against planted mistakes.

The mutation test copies ``oracle/oracle.c``, plants one plausible mistake (a
dropped term, a wrong sign, a transposed index, a missing reversal ...),
compiles the copy and requires that at least one pin fails on it.  Nothing is
planted in the repository's oracle itself.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)


SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement)
MUTATIONS = [
    ("drop_D_skip", "s->y_pre[i] = acc + Dd * xv;", "s->y_pre[i] = acc;"),
    ("exp_sign", "const double Abar = exp(dt * a);", "const double Abar = exp(-dt * a);"),
    ("drop_delta_in_Bbar", "Bbar = dt * Bt[n];", "Bbar = Bt[n];"),
    ("C_reads_B", "const double *Ct = s->C + (b * L + t) * N;", "const double *Ct = s->B + (b * L + t) * N;"),
    ("output_before_update", "h[n] = Abar * h[n] + Bbar * xv;\n            acc += Ct[n] * h[n];",
     "acc += Ct[n] * h[n];\n            h[n] = Abar * h[n] + Bbar * xv;"),
    ("A_transposed", "const double a = Arow[n];", "const double a = s->A[n * dim + d];"),
    ("ss2d_colmajor_transposed", "return (l % H) * W + l / H;", "return (l % W) * H + l / W;"),
    ("bidir_not_rereversed", "reverse_time(yr, y, batch, L, dim); /* back to token order */",
     "memcpy(y, yr, sizeof(double) * (size_t)tok);"),
    ("bidir_bwd_uses_fwd_params", "scan_t r = {xr, dr, A + dim * N,", "scan_t r = {xr, dr, A,"),
    ("softplus_wrong_branch", "return w > 0.0 ? w + log1p(exp(-w)) : log1p(exp(w));",
     "return w > 0.0 ? w + log1p(exp(w)) : log1p(exp(w));"),
    ("silu_sign", "if (z >= 0.0) return z / (1.0 + exp(-z));", "if (z >= 0.0) return z / (1.0 + exp(z));"),
    ("zoh_missing_divide", "Bbar = (a != 0.0 ? expm1(dt * a) / a : dt) * Bt[n];",
     "Bbar = (a != 0.0 ? expm1(dt * a) : dt) * Bt[n];"),
    ("bias_ignored", "if (s->delta_bias) dt += s->delta_bias[d];", ""),
    ("h0_ignored", "h[n] = s->h0 ? s->h0[(b * dim + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    # windowed cross-scan
    ("local_window_axes_swapped", "*row = (wi / nwx) * w + r / w;\n    *col = (wi % nwx) * w + r % w;",
     "*row = (wi / nwx) * w + r % w;\n    *col = (wi % nwx) * w + r / w;"),
    ("local_reversal_missing", "    int64_t r, c;\n    if (k >= 2) l = L - 1 - l;\n", "    int64_t r, c;\n"),
    ("local_window_rows_from_width", "*row = (wi / nwx) * w + r / w;", "*row = (wi / nwx) * w + (r / w + 1) % w;"),
    # backward
    ("bwd_adjoint_not_decayed", "            g[n] *= e;\n", ""),
    ("bwd_dA_missing_decay", "j->dA[d * N + n] += g[n] * (dt * e * hp[n] + dbda * Bt[n] * xv);",
     "j->dA[d * N + n] += g[n] * (dt * hp[n] + dbda * Bt[n] * xv);"),
    ("bwd_dB_missing_delta", "j->dB[(b * L + t) * N + n] += g[n] * beta * xv;", "j->dB[(b * L + t) * N + n] += g[n] * xv;"),
    ("bwd_dC_previous_state", "j->dC[(b * L + t) * N + n] += dyp * ht[n];", "j->dC[(b * L + t) * N + n] += dyp * hp[n];"),
    ("bwd_dx_missing_skip", "double dxv = Dd * dyp, ddt = 0.0;", "double dxv = 0.0, ddt = 0.0;"),
    ("bwd_ddelta_missing_input_term", "ddt += g[n] * (Arow[n] * e * hp[n] + dbdt * Bt[n] * xv);",
     "ddt += g[n] * (Arow[n] * e * hp[n]);"),
    # zero-order-hold backward
    ("bwd_zoh_input_term_not_decayed", "*dbeta_ddt = exp(y);", "*dbeta_ddt = 1.0;"),
    ("bwd_zoh_dA_input_term_dropped", "*dbeta_da = dt * dt * dphi;", "*dbeta_da = 0.0;"),
    ("bwd_zoh_dphi_series_weight", "dphi += (k + 1) * term / fact;", "dphi += term / fact;"),
    ("bwd_zoh_dphi_closed_form_sign", "dphi = (exp(y) * (y - 1.0) + 1.0) / (y * y);",
     "dphi = (exp(y) * (y + 1.0) - 1.0) / (y * y);"),
    ("bwd_zoh_euler_coefficient", "*beta = a != 0.0 ? expm1(y) / a : dt;", "*beta = dt;"),
    ("bwd_softplus_derivative_sign", "ddt * sigmoid(j->w[t])", "ddt * sigmoid(-j->w[t])"),
    ("bwd_silu_derivative_sign", "(1.0 + zv * (1.0 - sg))", "(1.0 - zv * (1.0 - sg))"),
    ("bwd_gate_not_applied", "dyp = s->dy[i] * zv * sg;", "dyp = s->dy[i];"),
    ("bwd_C_after_decay", "            g[n] += Ct[n] * dyp;\n", ""),
    ("bwd_h0_read_transposed", "for (int64_t n = 0; n < N; ++n) h[n] = s->h0 ? s->h0[(b * dim + d) * N + n] : 0.0;\n    const double Dd = s->D ? s->D[d] : 0.0;\n    const double *Arow = s->A + d * N;\n    for (int64_t t = 0; t < L; ++t) {\n        const int64_t i = (b * L + t) * dim + d;\n        double w",
     "for (int64_t n = 0; n < N; ++n) h[n] = s->h0 ? s->h0[(n * dim + d) % (s->batch * dim * N)] : 0.0;\n    const double Dd = s->D ? s->D[d] : 0.0;\n    const double *Arow = s->A + d * N;\n    for (int64_t t = 0; t < L; ++t) {\n        const int64_t i = (b * L + t) * dim + d;\n        double w"),
    ("conv1d_not_causal", "const int64_t s = t - (K - 1) + i;", "const int64_t s = t - (K - 1) / 2 + i;"),
    ("conv1d_filter_reversed", "v += w[d * K + i] * xv;", "v += w[d * K + (K - 1 - i)] * xv;"),
    ("conv1d_state_row_shifted",
     "else if (state_in) xv = state_in[(b * (K - 1) + (K - 1) + s) * dim + d];\n                    v += w",
     "else if (state_in) xv = state_in[(b * (K - 1) + (K - 2) + s) * dim + d];\n                    v += w"),
    ("conv1d_state_out_first_rows", "const int64_t s = L - (K - 1) + r;", "const int64_t s = r - (K - 1);"),
    ("conv1d_silu_skipped", "out[(b * L + t) * dim + d] = silu_ ? silu(v) : v;", "out[(b * L + t) * dim + d] = v;"),
    ("dwconv_kernel_transposed", "v += wt[(d * ks + i) * ks + j]", "v += wt[(d * ks + j) * ks + i]"),
    ("dwconv_no_centring", "const int64_t hh = h + i - p;", "const int64_t hh = h + i - p + (ks > 1);"),
    ("dwconv_bias_dropped", "double v = bias ? bias[d] : 0.0;\n                    for (int64_t i = 0; i < ks; ++i) {",
     "double v = 0.0;\n                    for (int64_t i = 0; i < ks; ++i) {"),
    # convolution backward
    ("conv_bwd_silu_derivative_sign", "return s * (1.0 + v * (1.0 - s));", "return s * (1.0 - v * (1.0 - s));"),
    ("conv1d_bwd_dx_tap_reversed", "dx[(b * L + s) * dim + d] += w[d * K + i] * dv;",
     "dx[(b * L + s) * dim + d] += w[d * K + (K - 1 - i)] * dv;"),
    ("conv1d_bwd_dw_missing_input", "dw[d * K + i] += xv * dv;", "dw[d * K + i] += dv;"),
    ("conv1d_bwd_state_rows_dropped",
     "if (dstate_in) dstate_in[(b * (K - 1) + (K - 1) + s) * dim + d] += w[d * K + i] * dv;", ""),
    ("conv1d_bwd_dbias_before_activation", "if (dbias) dbias[d] += dv;",
     "if (dbias) dbias[d] += dout[(b * L + t) * dim + d];"),
    ("dwconv_bwd_dx_kernel_transposed", "dx[q] += wt[(d * ks + i) * ks + j] * dv;",
     "dx[q] += wt[(d * ks + j) * ks + i] * dv;"),
    ("dwconv_bwd_dw_from_output_pixel", "dwt[(d * ks + i) * ks + j] += x[q] * dv;",
     "dwt[(d * ks + i) * ks + j] += x[((b * H + h) * W + w) * dim + d] * dv;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    text = open(SRC).read()
    assert old in text, f"mutation site for {name} not found in oracle.c"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new, 1))
    so = str(tmp_path / "libmutant.so")
    oracle.build(str(src), so)
    mutant = oracle.load(so)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
        except (RuntimeError, FloatingPointError, ValueError, OverflowError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")

# (name, function, text in oracle/__init__.py, replacement): mistakes in the compositions
# written in Python (multi-direction gradients out of the single-direction ones; scans along
# explicit orders).  The mutated function replaces the real one while its pin runs.
PY_MUTATIONS = [
    ("multi_dx_not_summed", "multi_bwd", 'out["dx"][:, o] += g["dx"]', 'out["dx"][:, o] = g["dx"]'),
    ("multi_dyp_not_gated", "multi_bwd", "dyp = dy * z * sg", "dyp = dy"),
    ("multi_dz_missing_silu_derivative", "multi_bwd", 'out["dz"] = dy * yp * sg * (1.0 + z * (1.0 - sg))',
     'out["dz"] = dy * yp * sg'),
    ("multi_first_direction_params", "multi_bwd", "A[k], B[k][:, o], C[k][:, o], dyp[:, o]",
     "A[0], B[k][:, o], C[k][:, o], dyp[:, o]"),
    ("multi_dC_not_scattered", "multi_bwd", 'out["dC"][k][:, o] = g["dC"]', 'out["dC"][k] = g["dC"]'),
    ("multi_ddelta_token_order", "multi_bwd", 'out["ddelta"][k][:, o] = g["ddelta"]', 'out["ddelta"][k] = g["ddelta"]'),
    ("ordered_not_scattered", "ordered_scan", "out[:, o] += yk", "out += yk"),
    ("ordered_gate_before_merge", "ordered_scan", "out *= z / (1.0 + np.exp(-z))", "out *= z / (1.0 + np.exp(z))"),
    ("ordered_delta_not_gathered", "ordered_scan", "yk = selscan(x[:, o], delta[k][:, o]",
     "yk = selscan(x[:, o], delta[k]"),
]
PY_PINS = {"multi_bwd": "pin_multi_bwd_fd", "ordered_scan": "pin_ordered_scan_maps"}


@pytest.mark.parametrize("name,fn,old,new", PY_MUTATIONS, ids=[m[0] for m in PY_MUTATIONS])
def test_pins_catch_planted_python_mistake(name, fn, old, new, lib, monkeypatch):
    text = open(PY_SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found once in oracle/__init__.py"
    ns = {"__name__": "oracle_mutant", "__file__": PY_SRC}
    exec(compile(text.replace(old, new, 1), PY_SRC, "exec"), ns)
    monkeypatch.setattr(oracle, fn, ns[fn])
    try:
        getattr(P, PY_PINS[fn])(lib)
    except AssertionError:
        return
    pytest.fail(f"no pin caught the planted mistake {name}")

