"""Planted mistakes: every plausible slip in the oracle must trip a pin.

Each mutant is a copy of ``oracle/mhc_oracle.cpp`` with one textual change
(a dropped term, a wrong sign, index or axis, a transposed operand, a swapped
map), compiled under a temporary directory on the CPU.  The test runs every
pin of ``oracle_pins`` against it and requires at least one to fail.
"""
import concurrent.futures as cf
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mhc_oracle.cpp")

MUTANTS = {
    "sinkhorn_rows_first": ("      if (h == 0) {", "      if (h == 1) {"),
    "sinkhorn_no_exp": ("M[i] = std::exp(logits[i]);", "M[i] = logits[i] + 5.0;"),
    "sinkhorn_one_pass_short": ("for (int t = 0; t < t_max; ++t) {", "for (int t = 0; t < t_max - 1; ++t) {"),
    "sinkhorn_column_by_row_sum": ("M[i * n + j] = M[i * n + j] / s[j];", "M[i * n + j] = M[i * n + j] / s[i];"),
    "rms_eps_outside_sqrt": ("std::sqrt(ss / K + eps)", "std::sqrt(ss / K) + eps"),
    "rms_mean_over_d": ("std::sqrt(ss / K + eps)", "std::sqrt(ss / d + eps)"),
    "rms_not_applied": ("acc += xh[k] *", "acc += x[k] *"),
    "phi_transposed": ("acc += xh[k] * static_cast<double>(phi[static_cast<int64_t>(k) * m + j]);",
                       "acc += xh[k] * static_cast<double>(phi[static_cast<int64_t>(j) * K + k]);"),
    "alpha_blocks_swapped": ("(j < n) ? alpha3[0] : (j < n + n * n) ? alpha3[1] : alpha3[2]",
                             "(j < n) ? alpha3[2] : (j < n + n * n) ? alpha3[1] : alpha3[0]"),
    "bias_dropped": ("out.logit[j] = a * out.z[j] + static_cast<double>(bias[j]);", "out.logit[j] = a * out.z[j];"),
    "read_map_doubled": ("out.H[i] = sigmoid(out.logit[i]);", "out.H[i] = 2.0 * sigmoid(out.logit[i]);"),
    "write_map_not_doubled": ("out.H[n + n * n + i] = 2.0 * sigmoid(", "out.H[n + n * n + i] = 1.0 * sigmoid("),
    "sigmoid_sign": ("return 1.0 / (1.0 + std::exp(-u));", "return 1.0 / (1.0 + std::exp(u));"),
    "tanh_gates": ("return 1.0 / (1.0 + std::exp(-u));", "return std::tanh(u);"),
    "mat_column_major": ("sinkhorn(n, &out.logit[n], t_max, &out.H[n], t_max > 0 ? trace.data() : nullptr);",
                         "std::vector<double> lt(n * n); for (int a = 0; a < n; ++a) for (int b = 0; b < n; ++b) "
                         "lt[a * n + b] = out.logit[n + b * n + a];\n"
                         "  sinkhorn(n, lt.data(), t_max, &out.H[n], t_max > 0 ? trace.data() : nullptr);"),
    "aggregate_wrong_flatten": ("acc += Hpre[i] * x[static_cast<int64_t>(i) * d + c];",
                                "acc += Hpre[i] * x[static_cast<int64_t>(c) * n + i];"),
    "aggregate_uses_post_map": ("if (h) aggregate(n, d, x, tm.H.data(), h + q * d);",
                                "if (h) aggregate(n, d, x, tm.H.data() + n + n * n, h + q * d);"),
    "mix_transposed": ("acc += Hres[i * n + j] * x[", "acc += Hres[j * n + i] * x["),
    "write_map_one_stream": ("acc + Hpost[i] * y[c];", "acc + Hpost[0] * y[c];"),
    "mix_drops_sublayer": ("acc + Hpost[i] * y[c];", "acc;"),
    "composite_right_multiply": ("acc += A[i * n + k] * P[k * n + j];", "acc += P[i * n + k] * A[k * n + j];"),
    "amax_rows_cols_swapped": ("rs += std::fabs(P[i * n + j]); cs += std::fabs(P[j * n + i]);",
                               "cs += std::fabs(P[i * n + j]); rs += std::fabs(P[j * n + i]);"),
    "amax_no_abs": ("rs += std::fabs(P[i * n + j]); cs += std::fabs(P[j * n + i]);",
                    "rs += P[i * n + j]; cs += P[j * n + i];"),
    "bf16_truncates": ("std::nearbyint(a / q) * q", "std::trunc(a / q) * q"),
    "gelu_wrong_cdf": ("std::erf(h / std::sqrt(2.0))", "std::tanh(h / std::sqrt(2.0))"),
    "bwd_rms_drops_radius_term": ("g.dx[k] += dxh[k] / tm.r + dr * x[k] / (K * tm.r);", "g.dx[k] += dxh[k] / tm.r;"),
    "bwd_sinkhorn_sign": ("dA[e] = (dM[e] - dot) / sm[a];", "dA[e] = (dM[e] + dot) / sm[a];"),
    "bwd_sinkhorn_forward_order": ("for (int st = 2 * t_max - 1; st >= 0; --st) {",
                                   "for (int st = 0; st < 2 * t_max; ++st) {"),
    "bwd_sinkhorn_no_exp_factor": ("for (int i = 0; i < nn; ++i) dM[i] *= M0[i];", ""),
    "bwd_write_gate_not_doubled": ("g.dH[n + n * n + i] * 2.0 * sq * (1.0 - sq);",
                                   "g.dH[n + n * n + i] * sq * (1.0 - sq);"),
    "bwd_mix_not_transposed": ("acc += Hres[i * n + j] * G[i * d + c];", "acc += Hres[j * n + i] * G[i * d + c];"),
    "bwd_alpha_from_logits": ("g.dalpha[blk] += g.dlogit[j] * tm.z[j];", "g.dalpha[blk] += g.dlogit[j] * tm.logit[j];"),
    "bwd_dz_without_alpha": ("g.dz[j] = static_cast<double>(alpha3[blk]) * g.dlogit[j];", "g.dz[j] = g.dlogit[j];"),
    "bwd_dphi_unnormalised": ("g.xhat[k] = x[k] / tm.r;", "g.xhat[k] = x[k];"),
    "bwd_dy_uses_read_map": ("acc += Hpost[i] * G[i * d + c];", "acc += Hpre[i] * G[i * d + c];"),
    "bwd_drops_aggregation": ("for (int c = 0; c < d; ++c) g.dx[i * d + c] += Hpre[i] * D[c];", ""),
    "bwd_dHres_transposed": ("acc += G[i * d + c] * x[j * d + c];", "acc += G[j * d + c] * x[i * d + c];"),
    "bwd_dHpre_uses_output_grad": ("for (int c = 0; c < d; ++c) acc += D[c] * x[i * d + c];",
                                   "for (int c = 0; c < d; ++c) acc += G[i * d + c] * x[i * d + c];"),
    "hc_no_tanh": ("H[j] = static_cast<double>(bias[j]) + a * std::tanh(tm.z[j]);",
                   "H[j] = static_cast<double>(bias[j]) + a * tm.z[j];"),
    "hc_alpha_inside_tanh": ("H[j] = static_cast<double>(bias[j]) + a * std::tanh(tm.z[j]);",
                             "H[j] = static_cast<double>(bias[j]) + std::tanh(a * tm.z[j]) * 1.5;"),
    "hc_drops_bias": ("H[j] = static_cast<double>(bias[j]) + a * std::tanh(tm.z[j]);", "H[j] = a * std::tanh(tm.z[j]);"),
    "stack_hc_uses_mhc_maps": ("if (kind == 1) return hc_maps(n, d, x, phi, bias, alpha3, eps);", ""),
    "stack_skips_rounding": ("for (int k = 0; k < K; ++k) x[k] = store_round(dtype, xo[k]);",
                             "for (int k = 0; k < K; ++k) x[k] = xo[k];"),
}


def _build_mutant(name, tmpdir):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} must appear exactly once"
    path = os.path.join(tmpdir, f"mut_{name}.cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    return oracle.build(force=True, src=path, out=os.path.join(tmpdir, f"libmut_{name}.so"))


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    tmpdir = str(tmp_path_factory.mktemp("oracle_mutants"))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        futs = {name: ex.submit(_build_mutant, name, tmpdir) for name in MUTANTS}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_libs):
    o = oracle.load(mutant_libs[name])
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
