"""Pins for the oracle's component-usage diagnostics (no GPU).

"Gaussian Mixture Attention: Linear-Time Sequence Mixing via Probabilistic
Latent Routing" proposes monitoring component under-use and collapse through
usage statistics of the responsibilities and the hard assignments
z_i = argmax_k gamma_ik (the discussion after the responsibility-gradient
identities, and the low-rank-affinity discussion); a companion page reports
components used and a normalised usage entropy, another gives per-token
responsibility entropy and a utilisation at gamma > 0.1.  The oracle is tied
to scikit-learn's posterior and scipy's entropy, and to closed cases.
"""
import numpy as np
import pytest
import scipy.stats

import oracle
from tests.test_oracle import _rand_problem, _sklearn_gamma


@pytest.mark.parametrize("seed,K,thr", [(0, 5, 0.1), (1, 9, 0.3), (2, 3, 0.0)])
def test_matches_sklearn_and_scipy(seed, K, thr):
    Q, _, _, mu, ls2, alpha = _rand_problem(seed, B=2, H=3, N=50, d_r=4, K=K)
    r = oracle.usage_stats(Q, mu, ls2, alpha, thr)
    G = _sklearn_gamma(Q, mu, ls2, alpha)                       # [B,H,N,K]
    T = 2 * 50
    np.testing.assert_allclose(r["mean_gamma"], G.sum(axis=(0, 2)) / T, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["utilization"], (G > thr).sum(axis=(0, 2)) / T)
    ent = scipy.stats.entropy(G, axis=-1)                       # nats, per token
    np.testing.assert_allclose(r["token_entropy"], ent.mean(axis=(0, 2)), rtol=1e-9)
    z = G.argmax(-1)
    for h in range(3):
        cnt = np.bincount(z[:, h].ravel(), minlength=K)
        np.testing.assert_array_equal(r["counts"][h], cnt)
        np.testing.assert_allclose(r["usage_entropy"][h],
                                   scipy.stats.entropy(cnt / T) / np.log(K), rtol=1e-12)
        assert r["used"][h] == np.count_nonzero(cnt)


def test_invariants():
    Q, _, _, mu, ls2, alpha = _rand_problem(3, B=3, H=2, N=40, d_r=5, K=7)
    r = oracle.usage_stats(Q, mu, ls2, alpha, 0.1)
    np.testing.assert_allclose(r["mean_gamma"].sum(-1), 1.0, rtol=1e-13)
    np.testing.assert_array_equal(r["counts"].sum(-1), 120)
    assert (r["token_entropy"] >= 0).all() and (r["token_entropy"] <= np.log(7) + 1e-12).all()
    assert (r["usage_entropy"] >= 0).all() and (r["usage_entropy"] <= 1 + 1e-12).all()


def test_identical_components_are_uniform():
    # equal means, variances and priors: gamma = 1/K for every token; the
    # argmax ties go to component 0
    rng = np.random.default_rng(4)
    K, d = 6, 3
    X = rng.standard_normal((1, 2, 30, d))
    mu = np.repeat(rng.standard_normal((2, 1, d)), K, axis=1)
    ls2 = np.repeat(rng.uniform(-1, 1, (2, 1, d)), K, axis=1)
    alpha = np.zeros((2, K))
    r = oracle.usage_stats(X, mu, ls2, alpha, 0.1)
    np.testing.assert_allclose(r["token_entropy"], np.log(K), rtol=1e-12)
    np.testing.assert_allclose(r["mean_gamma"], 1.0 / K, rtol=1e-12)
    np.testing.assert_allclose(r["utilization"], 1.0)             # 1/6 > 0.1
    np.testing.assert_array_equal(r["counts"][:, 0], 30)
    np.testing.assert_array_equal(r["used"], 1)
    np.testing.assert_array_equal(r["usage_entropy"], 0.0)
    assert (oracle.usage_stats(X, mu, ls2, alpha, 0.2)["utilization"] == 0).all()


def test_single_component():
    Q, _, _, mu, ls2, alpha = _rand_problem(5, B=2, H=2, N=17, d_r=3, K=1)
    r = oracle.usage_stats(Q, mu, ls2, alpha, 0.5)
    np.testing.assert_array_equal(r["counts"], 34)
    np.testing.assert_allclose(r["mean_gamma"], 1.0)
    np.testing.assert_allclose(r["token_entropy"], 0.0, atol=1e-15)
    np.testing.assert_array_equal(r["usage_entropy"], 0.0)


def test_separated_clusters_closed_form():
    # tokens placed at the means of well separated, narrow components: one-hot
    # responsibilities, counts equal to the construction
    K, d = 4, 2
    mu = np.array([[[0.0, 0.0], [40.0, 0.0], [0.0, 40.0], [40.0, 40.0]]])
    ls2 = np.full((1, K, d), -2.0)
    alpha = np.zeros((1, K))
    sizes = [5, 0, 9, 2]
    X = np.concatenate([np.repeat(mu[0, k][None], n, 0) for k, n in enumerate(sizes)])[None, None]
    X = X + 1e-3 * np.random.default_rng(6).standard_normal(X.shape)
    r = oracle.usage_stats(X, mu, ls2, alpha, 0.1)
    np.testing.assert_array_equal(r["counts"][0], sizes)
    assert r["used"][0] == 3
    p = np.array(sizes) / 16.0
    p = p[p > 0]
    np.testing.assert_allclose(r["usage_entropy"][0], -(p * np.log(p)).sum() / np.log(K),
                               rtol=1e-12)
    np.testing.assert_allclose(r["token_entropy"][0], 0.0, atol=1e-12)
    np.testing.assert_allclose(r["utilization"][0], p_full := np.array(sizes) / 16.0)
    np.testing.assert_allclose(r["mean_gamma"][0], p_full, atol=1e-12)
