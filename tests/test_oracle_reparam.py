"""Pins for the oracle's parameter reparameterisation (no GPU).

Eq. 14 of "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
Probabilistic Latent Routing" (the reparameterisations used for training) sets
sigma^2 = log(1 + exp(omega)) + eps_sigma; Eq. 15 sets pi = softmax(alpha).
The oracle's log sigma^2 and log pi are checked against scipy's softplus and
log_softmax (routines the oracle does not call), closed values, and the
invariants of the softmax.
"""
import numpy as np
import pytest
import scipy.special as sps

import oracle


def _params(seed, H=3, K=7, d_r=5, scale=4.0):
    rng = np.random.default_rng(seed)
    return rng.normal(0, scale, (H, K, d_r)), rng.normal(0, scale, (H, K))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_scipy(seed):
    om, al = _params(seed)
    r = oracle.reparameterize(om, al, 1e-4)
    np.testing.assert_allclose(r["log_sigma2"], np.log(sps.softplus(om) + 1e-4), rtol=1e-13)
    np.testing.assert_allclose(r["log_pi"], sps.log_softmax(al, axis=-1), rtol=1e-13,
                               atol=1e-13)


def test_closed_values():
    om = np.array([[[0.0, np.log(np.e - 1.0), 800.0, -800.0]]])
    al = np.array([[0.0, 0.0, np.log(2.0)]])
    r = oracle.reparameterize(om, al, 0.5)
    # softplus(0) = log 2; softplus(log(e - 1)) = 1; large w: w; very negative: 0
    np.testing.assert_allclose(r["log_sigma2"][0, 0],
                               np.log([np.log(2.0) + 0.5, 1.5, 800.5, 0.5]), rtol=1e-14)
    # priors 1/4, 1/4, 1/2
    np.testing.assert_allclose(np.exp(r["log_pi"][0]), [0.25, 0.25, 0.5], rtol=1e-14)


def test_softmax_invariants():
    om, al = _params(3, K=11)
    r = oracle.reparameterize(om, al, 1e-3)
    # the priors lie on the simplex; shifting all logits of a head changes nothing
    np.testing.assert_allclose(np.exp(r["log_pi"]).sum(-1), 1.0, rtol=1e-14)
    r2 = oracle.reparameterize(om, al + np.array([[5.0], [-300.0], [1e3]]), 1e-3)
    np.testing.assert_allclose(r2["log_pi"], r["log_pi"], atol=1e-12)
    # the variance floor: sigma^2 >= eps_sigma, strictly increasing in omega
    s2 = np.exp(r["log_sigma2"])
    assert (s2 > 1e-3).all()
    w = np.linspace(-30, 30, 101)[None, None, :]
    ls = oracle.reparameterize(w, np.zeros((1, 1)), 1e-3)["log_sigma2"][0, 0]
    assert (np.diff(ls) > 0).all()


def test_forward_posterior_independent_of_logit_shift():
    # the forward takes log pi up to a per-head constant: alpha itself and
    # log softmax(alpha) give the same output
    rng = np.random.default_rng(4)
    B, H, N, d_r, d_v, K = 1, 2, 9, 4, 3, 5
    Q, Kx = rng.normal(size=(B, H, N, d_r)), rng.normal(size=(B, H, N, d_r))
    V = rng.normal(size=(B, H, N, d_v))
    mu = rng.normal(size=(H, K, d_r))
    om, al = rng.normal(size=(H, K, d_r)), rng.normal(size=(H, K))
    r = oracle.reparameterize(om, al, 1e-4)
    o1 = oracle.forward(Q, Kx, V, mu, r["log_sigma2"], r["log_pi"], 1e-6, False)["out"]
    o2 = oracle.forward(Q, Kx, V, mu, r["log_sigma2"], al, 1e-6, False)["out"]
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
