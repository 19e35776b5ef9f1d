"""Mutation check of the oracle's pins (no GPU).

Each case plants one plausible mistake in a copy of oracle/hstu_oracle.c (a
flipped sign or index, a dropped term, a transposed operand, a wrong
normaliser), builds it, and requires that at least one pin of
tests/test_oracle_pins.py fails on it.  The real oracle is never modified.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "hstu_oracle.c")

# (name, text to replace, replacement); each text must occur in the source.
MUTANTS = [
    ("position-sign", "int64_t r = j - i;", "int64_t r = i - j;"),
    ("silu-sign", "static double silu(double s) { return s / (1.0 + exp(-s)); }",
     "static double silu(double s) { return s / (1.0 + exp(s)); }"),
    ("drop-time-bias", "if (rab_t && have_t) s +=", "if (0) s +="),
    ("bucket-no-plus-one", "floor_log2_u64(mag + 1u)", "floor_log2_u64(mag)"),
    ("strict-causal", "for (int64_t j = 0; j <= i; j++) {\n            int64_t rk = o_b + j;\n            double s",
     "for (int64_t j = 0; j < i; j++) {\n            int64_t rk = o_b + j;\n            double s"),
    ("wrong-normaliser", "for (int c = 0; c < dv; c++) acc[c] /= (double)N;",
     "for (int c = 0; c < dv; c++) acc[c] /= (double)(N + 1);"),
    ("key-from-query-row", "k + (rk * H + h) * dqk, dqk, i, j", "k + (r * H + h) * dqk, dqk, i, j"),
    ("unbiased-variance", "        var /= F;\n        double rstd = 1.0 / sqrt(var + eps);\n        for (int c = 0; c < F; c++) G",
     "        var /= (F - 1);\n        double rstd = 1.0 / sqrt(var + eps);\n        for (int c = 0; c < F; c++) G"),
    ("silu-grad", "return sg * (1.0 + s * (1.0 - sg));", "return sg * (1.0 + s * sg);"),
    ("dq-transposed-operand", "dq[(r * H + h) * dqk + c] += ds * kj[c];", "dq[(r * H + h) * dqk + c] += ds * qi[c];"),
    ("dv-missing-scale", "+= p * doi[c] / (double)N;", "+= p * doi[c];"),
    ("ln-bwd-dropped-mean", "dO[r * F + c] = rstd * (dxh - m1 - xh * m2);", "dO[r * F + c] = rstd * (dxh - xh * m2);"),
    ("rab-head-stride", "s += rab_p[(int64_t)h * (2 * N + 1) +", "s += rab_p[(int64_t)h * (2 * N) +"),
    ("split-order-uv", "Um[r * HD + c] = A[r * Z4 + c];\n            Vm[r * HD + c] = A[r * Z4 + HD + c];",
     "Um[r * HD + c] = A[r * Z4 + HD + c];\n            Vm[r * HD + c] = A[r * Z4 + c];"),
    ("split-order-qk", "Qm[r * HD + c] = A[r * Z4 + 2 * HD + c];\n            Km[r * HD + c] = A[r * Z4 + 3 * HD + c];",
     "Qm[r * HD + c] = A[r * Z4 + 3 * HD + c];\n            Km[r * HD + c] = A[r * Z4 + 2 * HD + c];"),
    ("no-residual", "Y[r * D + n] = X[r * D + n] + y;", "Y[r * D + n] = y;"),
    ("mfalcon-position", "d, nu, j, N, h, rp, rt,", "d, nu - 1, j, N, h, rp, rt,"),
    ("mfalcon-no-self", "acc[e] = (acc[e] + p * vv[h * d + e]) / (double)N;", "acc[e] = acc[e] / (double)N;"),
    ("mfalcon-self-time", "rp, rt, 0, 0,\n", "rp, rt, 0, 1,\n"),
    ("drab-t-sign", "oracle_time_bucket(ts[r] - ts[rk])] += ds;", "oracle_time_bucket(ts[r] - ts[rk])] -= ds;"),
    ("layer-bwd-no-residual", "double s = dY[r * D + c];", "double s = 0.0;"),
    ("layer-bwd-sigmoid-for-silu-grad", "(z > 0.0 ? 1.0 : 0.0) : silu_grad(z); }", "(z > 0.0 ? 1.0 : 0.0) : 1.0 / (1.0 + exp(-z)); }"),
    ("layer-bwd-dw1-wrong-operand", "s += dA[r * Z4 + n] * X[r * D + c];", "s += dA[r * Z4 + n] * dY[r * D + c];"),
    ("layer-bwd-dw2-ungated", "s += dY[r * D + n] * G[r * HD + c];", "s += dY[r * D + n] * Um[r * HD + c];"),
    ("layer-bwd-dg-transposed-w2", "s += dY[r * D + n] * W2[(int64_t)n * HD + c];", "s += dY[r * D + n] * W2[(int64_t)c * D + n];"),
    ("layer-bwd-dq-dk-swapped", "dA[r * Z4 + 2 * HD + c] = dq[r * HD + c];", "dA[r * Z4 + 2 * HD + c] = dk[r * HD + c];"),
    ("append-position", "int64_t pos = nu + i;", "int64_t pos = nu + i + 1;"),
    ("append-strict-causal", "for (int64_t i2 = 0; i2 <= i; i2++)", "for (int64_t i2 = 0; i2 < i; i2++)"),
    ("append-no-history", "for (int64_t j = 0; j < nu; j++) { /* the cached history */",
     "for (int64_t j = 0; j < nu - 1; j++) { /* the cached history */"),
    ("append-merged-offset", "int64_t mo = ho + ao;", "int64_t mo = ho;"),
    ("softmax-no-scale", "double scale = 1.0 / sqrt((double)dqk);", "double scale = 1.0;"),
    ("softmax-strict-causal", "for (int64_t j = 0; j <= i; j++) {\n            double x = 0.0;",
     "for (int64_t j = 0; j < i; j++) {\n            double x = 0.0;"),
    ("softmax-no-denominator", "for (int c = 0; c < dv; c++) acc[c] /= den;", "for (int c = 0; c < dv; c++) acc[c] /= 1.0;"),
    ("sl-floor-length", "double x = ceil((double)n * pow(u[b], 1.0 / alpha));",
     "double x = floor((double)n * pow(u[b], 1.0 / alpha));"),
    ("sl-ties-reversed", "(keys[o + i] == keys[o + j] && i < j)", "(keys[o + i] == keys[o + j] && i > j)"),
    ("sl-largest-keys", "if (keys[o + i] < keys[o + j] ||", "if (keys[o + i] > keys[o + j] ||"),
    ("append-new-time", "have_t ? add_ts[r] : 0, have_t ? add_ts[rk] : 0, have_t);",
     "have_t ? add_ts[r] : 0, have_t ? add_ts[r] : 0, have_t);"),
]

PINS = [
    (pins.test_fwd_matches_dense_bruteforce, dict(seed=0)),
    (pins.test_fwd_matches_dense_bruteforce, dict(seed=1)),
    (pins.test_fwd_matches_dense_bruteforce, dict(seed=2)),
    (pins.test_fwd_tiny_layer_workload_matches_dense, {}),
    (pins.test_layer_matches_dense_strong_branch, dict(phi1=0)),
    (pins.test_closed_form_prefix_sum, {}),
    (pins.test_closed_form_single_token, {}),
    (pins.test_bias_readout_closed_form, {}),
    (pins.test_time_bucket_exhaustive_and_powers, {}),
    (pins.test_ln_gate_against_library_and_moments, {}),
    (pins.test_bwd_finite_differences, dict(with_u=True)),
    (pins.test_bwd_identities, {}),
    (pins.test_mfalcon_equals_last_row_of_full_forward, {}),
    (pins.test_layer_bwd_residual_and_bias_identities, {}),
    (pins.test_layer_bwd_finite_differences, dict(phi1=0)),
    (pins.test_layer_append_equals_full_forward, {}),
    (pins.test_softmax_comparator_against_library_softmax, {}),
    (pins.test_softmax_comparator_closed_forms, {}),
    (pins.test_sl_sample_selection_definition, {}),
]


def _pins_fail() -> bool:
    for fn, kw in PINS:
        try:
            fn(**kw)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new, 1)
    cpath = os.path.join(tmp_path, "mut.c")
    lpath = os.path.join(tmp_path, "libmut.so")
    with open(cpath, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lpath, cpath, "-lm"])
    old_lib = oracle.swap_library(lpath)
    try:
        assert _pins_fail(), "mutant survived every pin: " + name
    finally:
        oracle.swap_library(None)
        oracle._load()


def test_real_oracle_passes_the_same_pins():
    assert not _pins_fail()
