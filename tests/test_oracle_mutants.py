"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them: evidence that the pins constrain each part
of the definition, not only the oracle's own formula."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
import pins  # noqa: E402

SRC = os.path.join(os.path.dirname(oracle.__file__), "la_oracle.c")

# (name, original text, mutated text): each must occur exactly once
MUTANTS = [
    # softmax attention layer
    ("sm_diagonal_excluded", "const int64_t last = t;", "const int64_t last = t - 1;"),
    ("sm_rope_direction", "y[2 * i + 1] = a * s + b * c;", "y[2 * i + 1] = -a * s + b * c;"),
    ("sm_rope_frequency", "pow(base, -2.0 * (double)i / (double)rope_dim)",
     "pow(base, -(double)i / (double)rope_dim)"),
    ("sm_rope_query_position_global",
     "rope_vec(q + (t * H + h) * D, qh, D, rope_dim, base, (double)(t - s0));",
     "rope_vec(q + (t * H + h) * D, qh, D, rope_dim, base, (double)t);"),
    ("sm_scale_missing", "p[u - s0] = scale * dot;", "p[u - s0] = dot;"),
    ("sm_normaliser_missing", "o[j] = acc / z;", "o[j] = acc;"),
    ("sm_passthrough_dropped", "for (int64_t j = rope_dim; j < D; ++j) y[j] = x[j];",
     "for (int64_t j = rope_dim; j < D; ++j) y[j] = 0.0;"),
    ("sm_keys_across_sequences", "const int64_t s0 = seg[s];\n            double* qh",
     "const int64_t s0 = 0;\n            double* qh"),
    ("diagonal_excluded",
     "                /* state update first: the current token attends to itself */\n"
     "                for (int64_t i = 0; i < D; ++i)\n"
     "                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += kt[i] * vt[j];\n"
     "                /* y_t = q~_t S */\n"
     "                for (int64_t j = 0; j < D; ++j) {\n"
     "                    double acc = 0.0;\n"
     "                    for (int64_t i = 0; i < D; ++i) acc += qt[i] * S[i * D + j];\n"
     "                    out[base + j] = acc;\n"
     "                }\n",
     "                for (int64_t j = 0; j < D; ++j) {\n"
     "                    double acc = 0.0;\n"
     "                    for (int64_t i = 0; i < D; ++i) acc += qt[i] * S[i * D + j];\n"
     "                    out[base + j] = acc;\n"
     "                }\n"
     "                for (int64_t i = 0; i < D; ++i)\n"
     "                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += kt[i] * vt[j];\n"),
    ("state_transposed",
     "for (int64_t j = 0; j < D; ++j) S[i * D + j] += kt[i] * vt[j];\n                /* y_t",
     "for (int64_t j = 0; j < D; ++j) S[i * D + j] += kt[j] * vt[i];\n                /* y_t"),
    ("norm_sum_not_mean", "sqrt(ss / (double)HD + eps)", "sqrt(ss + eps)"),
    ("eps_outside_sqrt", "sqrt(ss / (double)HD + eps)", "(sqrt(ss / (double)HD) + eps)"),
    ("gate_silu", "y[i] * r * w[i] * sigmoid(g[i])", "y[i] * r * w[i] * silu(g[i])"),
    ("gate_missing", "y[i] * r * w[i] * sigmoid(g[i])", "y[i] * r * w[i]"),
    ("weight_per_dim", "y[i] * r * w[i] * sigmoid(g[i])", "y[i] * r * w[i % 2] * sigmoid(g[i])"),
    ("no_silu_on_v", "vt[i] = silu(v[base + i]);", "vt[i] = v[base + i];"),
    ("sigmoid_sign", "1.0 / (1.0 + exp(-x))", "1.0 / (1.0 + exp(x))"),
    ("init_state_ignored",
     "            if (init_state) memcpy(S, init_state + (s * H + h) * D * D, sizeof(double) * D * D);\n"
     "            else memset(S, 0, sizeof(double) * D * D);\n"
     "            for (int64_t t = seg[s]",
     "            memset(S, 0, sizeof(double) * D * D);\n"
     "            for (int64_t t = seg[s]"),
    ("init_state_wrong_segment",
     "            if (init_state) memcpy(S, init_state + (s * H + h) * D * D, sizeof(double) * D * D);\n"
     "            else memset(S, 0, sizeof(double) * D * D);\n"
     "            for (int64_t t = seg[s]",
     "            if (init_state) memcpy(S, init_state + h * D * D, sizeof(double) * D * D);\n"
     "            else memset(S, 0, sizeof(double) * D * D);\n"
     "            for (int64_t t = seg[s]"),
    ("decode_uses_old_state",
     "                for (int64_t j = 0; j < D; ++j) S[i * D + j] += silu(k[base + i]) * silu(v[base + j]);\n"
     "            for (int64_t j = 0; j < D; ++j) {\n"
     "                double acc = 0.0;\n"
     "                for (int64_t i = 0; i < D; ++i) acc += silu(q[base + i]) * S[i * D + j];\n"
     "                out[base + j] = acc;\n"
     "            }\n",
     "                ;\n"
     "            for (int64_t j = 0; j < D; ++j) {\n"
     "                double acc = 0.0;\n"
     "                for (int64_t i = 0; i < D; ++i) acc += silu(q[base + i]) * S[i * D + j];\n"
     "                out[base + j] = acc;\n"
     "            }\n"
     "            for (int64_t i = 0; i < D; ++i)\n"
     "                for (int64_t j = 0; j < D; ++j) S[i * D + j] += silu(k[base + i]) * silu(v[base + j]);\n"),
    ("blocked_mask_strict", "for (int64_t c = 0; c <= a; ++c)", "for (int64_t c = 0; c < a; ++c)"),
    # backward
    ("bwd_norm_mean_term_dropped", "dy[e] = r * (a - yhat[e] * ay / (double)HD);", "dy[e] = r * a;"),
    ("bwd_dq_state_not_transposed", "acc += dy[base + j] * S[i * D + j];",
     "acc += dy[base + j] * S[j * D + i];"),
    ("bwd_dk_uses_k", "acc += S[i * D + j] * vt[j];", "acc += S[i * D + j] * kt[j];"),
    ("bwd_dv_silu_grad_missing", "dv[base + j] = acc * silu_grad(v[base + j]);", "dv[base + j] = acc;"),
    ("bwd_gate_derivative", "dg[e] = dout[e] * yhat[e] * w[i] * sg * (1.0 - sg);",
     "dg[e] = dout[e] * yhat[e] * w[i] * sg;"),
    ("bwd_dw_without_gate", "acc += dout[t * HD + i] * yhat[t * HD + i] * sigmoid(g[t * HD + i]);",
     "acc += dout[t * HD + i] * yhat[t * HD + i];"),
    ("bwd_final_state_gradient_ignored",
     "            if (d_final) memcpy(S, d_final + (s * H + h) * D * D, sizeof(double) * D * D);\n"
     "            else memset(S, 0, sizeof(double) * D * D);\n",
     "            memset(S, 0, sizeof(double) * D * D);\n"),
    ("bwd_state_gradient_one_token_late",
     "                for (int64_t i = 0; i < D; ++i)\n"
     "                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += qt[i] * dy[base + j];\n"
     "                for (int64_t i = 0; i < D; ++i) {\n"
     "                    double acc = 0.0;\n"
     "                    for (int64_t j = 0; j < D; ++j) acc += S[i * D + j] * vt[j];\n"
     "                    dk[base + i] = acc * silu_grad(k[base + i]);\n"
     "                }\n",
     "                for (int64_t i = 0; i < D; ++i) {\n"
     "                    double acc = 0.0;\n"
     "                    for (int64_t j = 0; j < D; ++j) acc += S[i * D + j] * vt[j];\n"
     "                    dk[base + i] = acc * silu_grad(k[base + i]);\n"
     "                }\n"
     "                for (int64_t i = 0; i < D; ++i)\n"
     "                    for (int64_t j = 0; j < D; ++j) S[i * D + j] += qt[i] * dy[base + j];\n"),
]


def _build_mutant(tmpdir, orig, new):
    src = open(SRC).read()
    assert src.count(orig) == 1, "mutation anchor must occur once: %r" % orig[:60]
    path = os.path.join(tmpdir, "m.c")
    with open(path, "w") as f:
        f.write(src.replace(orig, new))
    so = os.path.join(tmpdir, "libm.so")
    subprocess.run(["gcc", "-O1", "-std=gnu99", "-fopenmp", "-fPIC", "-shared", path, "-o", so,
                    "-lm"], check=True)
    return so


@pytest.mark.parametrize("name,orig,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, new):
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    tmp = tempfile.mkdtemp(prefix="la_mut_")
    try:
        so = _build_mutant(tmp, orig, new)
        saved = oracle._load()
        oracle._lib = oracle._bind(so)
        failed = []
        try:
            for pin in pins.ALL_PINS:
                try:
                    pin(oracle)
                except AssertionError:
                    failed.append(pin.__name__)
        finally:
            oracle._lib = saved
        assert failed, "no pin caught the planted mistake %s" % name
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
