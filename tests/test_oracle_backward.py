"""Pins for the oracle's backward pass (no GPU).

The gradients follow "Gradient structure" of "Gaussian Mixture Attention:
Linear-Time Sequence Mixing via Probabilistic Latent Routing" (the score
gradient of Eq. 18).  They are tied to the C forward, which is pinned on its
own: central finite differences of L = sum(dO * O) in fp64 must match every
gradient; plus invariants of the score (a common shift of routing vectors and
means, a per-head constant in log pi) and the single-component case.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle import _rand_problem


def _loss(Q, Kx, V, mu, ls2, lpi, eps, dO, causal=False):
    return float((oracle.forward(Q, Kx, V, mu, ls2, lpi, eps, causal)["out"] * dO).sum())


def _fd(fun, x, idx, h=1e-6):
    xp = x.copy()
    xm = x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (fun(xp) - fun(xm)) / (2 * h)


@pytest.mark.parametrize("seed,causal", [(0, False), (1, False), (0, True), (1, True)])
def test_gradients_match_finite_differences(seed, causal):
    Q, Kx, V, mu, ls2, lpi = _rand_problem(seed, B=2, H=2, N=7, d_r=3, d_v=4, K=4)
    eps = 1e-3
    dO = np.random.default_rng(seed + 10).standard_normal(V.shape)
    g = oracle.backward(Q, Kx, V, mu, ls2, lpi, eps, dO, causal)
    args = dict(Q=Q, Kx=Kx, V=V, mu=mu, ls2=ls2, lpi=lpi)
    names = {"Q": "dQ", "Kx": "dK", "V": "dV", "mu": "dmu", "ls2": "dlog_sigma2",
             "lpi": "dlog_pi"}
    rng = np.random.default_rng(seed + 20)
    for arg, gname in names.items():
        x = args[arg]
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)

            def fun(xv, arg=arg):
                a = dict(args)
                a[arg] = xv
                return _loss(a["Q"], a["Kx"], a["V"], a["mu"], a["ls2"], a["lpi"], eps, dO,
                             causal)
            fd = _fd(fun, x, idx)
            assert abs(g[gname][idx] - fd) <= 1e-6 * (1 + abs(fd)), (gname, idx, g[gname][idx], fd)


def test_score_invariances():
    Q, Kx, V, mu, ls2, lpi = _rand_problem(2, B=2, H=3, N=9, d_r=4, d_v=3, K=5)
    dO = np.random.default_rng(3).standard_normal(V.shape)
    g = oracle.backward(Q, Kx, V, mu, ls2, lpi, 1e-6, dO)
    # log pi enters only through a softmax: its gradient sums to zero per head
    np.testing.assert_allclose(g["dlog_pi"].sum(-1), 0.0, atol=1e-12)
    # the scores depend on x - mu only: a common shift of every routing vector
    # and mean of a head leaves the loss unchanged, so the gradients cancel
    tot = g["dQ"].sum(axis=(0, 2)) + g["dK"].sum(axis=(0, 2)) + g["dmu"].sum(axis=1)
    np.testing.assert_allclose(tot, 0.0, atol=1e-11)


def test_single_component_gradients():
    # K = 1: gamma = 1 everywhere, the output is the mean of V scaled by
    # N / (N + eps); no gradient reaches the routing side
    Q, Kx, V, mu, ls2, lpi = _rand_problem(4, B=1, H=2, N=6, d_r=3, d_v=2, K=1)
    eps = 0.5
    dO = np.random.default_rng(5).standard_normal(V.shape)
    g = oracle.backward(Q, Kx, V, mu, ls2, lpi, eps, dO)
    for k in ("dQ", "dK", "dmu", "dlog_sigma2", "dlog_pi"):
        np.testing.assert_allclose(g[k], 0.0, atol=1e-13)
    np.testing.assert_allclose(g["dV"], np.broadcast_to(dO.sum(2, keepdims=True) / (6 + eps),
                                                        V.shape), rtol=1e-13)


def test_causal_last_position_gradient_is_bidirectional():
    # a loss on the last position only: the causal and bidirectional forwards
    # agree there, and so do all gradients
    Q, Kx, V, mu, ls2, lpi = _rand_problem(6, B=1, H=2, N=8, d_r=3, d_v=2, K=3)
    dO = np.zeros(V.shape)
    dO[:, :, -1] = np.random.default_rng(7).standard_normal(dO[:, :, -1].shape)
    gc = oracle.backward(Q, Kx, V, mu, ls2, lpi, 1e-6, dO, True)
    gb = oracle.backward(Q, Kx, V, mu, ls2, lpi, 1e-6, dO, False)
    for k in gc:
        np.testing.assert_allclose(gc[k], gb[k], rtol=1e-11, atol=1e-13)


def test_causal_future_dO_does_not_reach_the_past_values():
    # dO at position i reaches only values at j <= i
    Q, Kx, V, mu, ls2, lpi = _rand_problem(8, B=1, H=1, N=9, d_r=2, d_v=3, K=3)
    dO = np.zeros(V.shape)
    dO[:, :, 4] = 1.0
    g = oracle.backward(Q, Kx, V, mu, ls2, lpi, 1e-6, dO, True)
    assert np.all(g["dV"][:, :, 5:] == 0) and np.all(g["dK"][:, :, 5:] == 0)
    assert np.all(g["dQ"][:, :, :4] == 0) and np.all(g["dQ"][:, :, 5:] == 0)
