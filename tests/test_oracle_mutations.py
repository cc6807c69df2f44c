"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case compiles a copy of oracle/gma_oracle.c with one plausible slip (a
dropped term, a wrong sign or index, an exclusive instead of inclusive causal
prefix, a different tie rule) and checks that at least one pin of
test_oracle.py's kind fails against it.  The pristine source must pass the
same battery.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.test_oracle import _rand_problem, _sklearn_gamma, _sklearn_gmm

SRC = os.path.join(os.path.dirname(oracle.__file__), "gma_oracle.c")

MUTATIONS = {
    "drop_logdet": ("q += diff * diff / var + ls2[(size_t)k * d_r + d] + GMAO_LOG_2PI;",
                    "q += diff * diff / var + GMAO_LOG_2PI;"),
    "wrong_sign_quadratic": ("s[k] = logpi[k] - 0.5 * q;", "s[k] = logpi[k] + 0.5 * q;"),
    "drop_prior": ("s[k] = logpi[k] - 0.5 * q;", "s[k] = -0.5 * q;"),
    "std_for_variance": ("double var = exp(ls2[(size_t)k * d_r + d]);",
                         "double var = exp(0.5 * ls2[(size_t)k * d_r + d]);"),
    "transposed_mean_index": ("double diff = x[d] - mu[(size_t)k * d_r + d];",
                              "double diff = x[d] - mu[(size_t)d * K + k];"),
    "plus_mean": ("double diff = x[d] - mu[(size_t)k * d_r + d];",
                  "double diff = x[d] + mu[(size_t)k * d_r + d];"),
    "tie_to_highest": ("if (s[k] > m) { m = s[k]; arg = k; }",
                       "if (s[k] >= m) { m = s[k]; arg = k; }"),
    "unnormalised_gamma": ("for (int k = 0; k < K; ++k) gamma[k] /= tot;",
                           "for (int k = 0; k < K; ++k) gamma[k] /= 1.0;"),
    "no_eps": ("den += j->eps;", "den += 0.0;"),
    "write_from_queries": ("scores(kx + (size_t)t * d_r, d_r, mu, ls2, logpi, K, s);",
                           "scores(q + (size_t)t * d_r, d_r, mu, ls2, logpi, K, s);"),
    "causal_exclusive_prefix": (
        "int want = j->rows ? (r < nout && j->rows[r] == i) : 1;",
        "for (int k = 0; k < K; ++k) { z[k] -= gk[k]; for (int e = 0; e < d_v; ++e)"
        " vt[(size_t)k * d_v + e] -= gk[k] * v[(size_t)i * d_v + e]; }\n"
        "      int want = j->rows ? (r < nout && j->rows[r] == i) : 1;"),
    "causal_query_reads_key": (
        "scores(q + (size_t)i * d_r, d_r, mu, ls2, logpi, K, s);\n      int32_t aq",
        "scores(kx + (size_t)i * d_r, d_r, mu, ls2, logpi, K, s);\n      int32_t aq"),
}


def _battery():
    """A quick subset of the pins; raises AssertionError on the first miss."""
    eps = 1e-6
    # responsibilities and raw scores against scikit-learn
    Q, Kx, V, mu, ls2, alpha = _rand_problem(21, B=1, H=2, N=96, K=5)
    r = oracle.responsibilities(Q, mu, ls2, alpha)
    np.testing.assert_allclose(r["gamma"], _sklearn_gamma(Q, mu, ls2, alpha), atol=1e-10)
    gm = _sklearn_gmm(mu[0], ls2[0], alpha[0])
    np.testing.assert_allclose(r["score"][0, 0], gm._estimate_weighted_log_prob(Q[0, 0]),
                               rtol=1e-12, atol=1e-9)
    # brute-force affinity, both variants
    GQ = _sklearn_gamma(Q, mu, ls2, alpha)
    GK = _sklearn_gamma(Kx, mu, ls2, alpha)
    for causal in (False, True):
        A = np.einsum("bhik,bhjk->bhij", GQ, GK)
        if causal:
            A = A * np.tril(np.ones(A.shape[-2:]))
        expect = np.einsum("bhij,bhjd->bhid", A, V) / (A.sum(-1, keepdims=True) + eps)
        got = oracle.forward(Q, Kx, V, mu, ls2, alpha, eps, causal)["out"]
        np.testing.assert_allclose(got, expect, rtol=1e-9, atol=1e-12)
    # K = 1 closed forms
    Q, Kx, V, mu, ls2, alpha = _rand_problem(22, B=1, H=1, N=50, K=1)
    N = 50
    got = oracle.forward(Q, Kx, V, mu, ls2, alpha, eps, False)["out"]
    np.testing.assert_allclose(got, np.broadcast_to(V.sum(2, keepdims=True) / (N + eps), V.shape),
                               rtol=1e-12)
    got = oracle.forward(Q, Kx, V, mu, ls2, alpha, eps, True)["out"]
    cnt = np.arange(1, N + 1, dtype=np.float64)[None, None, :, None]
    np.testing.assert_allclose(got, np.cumsum(V, 2) / (cnt + eps), rtol=1e-12)
    # exact tie goes to the lowest index
    rng = np.random.default_rng(23)
    mu = np.repeat(rng.standard_normal((1, 1, 4)), 3, axis=1)
    ls2 = np.zeros((1, 3, 4))
    a = oracle.responsibilities(rng.standard_normal((1, 20, 4)), mu, ls2, np.zeros((1, 3)))
    np.testing.assert_array_equal(a["assign"], 0)


def _compile(src_text, tmp_path, name):
    c = tmp_path / (name + ".c")
    c.write_text(src_text)
    so = tmp_path / (name + ".so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c),
                           "-lm", "-lpthread"])
    return str(so)


def test_pristine_source_passes_battery(tmp_path):
    so = _compile(open(SRC).read(), tmp_path, "pristine")
    with oracle.using_library(so):
        _battery()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after = MUTATIONS[name]
    text = open(SRC).read()
    assert before in text, "mutation anchor no longer present: " + name
    so = _compile(text.replace(before, after), tmp_path, name)
    with oracle.using_library(so):
        with pytest.raises(AssertionError):
            _battery()
