"""Pins for the oracle's causal decode step (no GPU).

The decode step appends one token to a carried prefix state ("Causal GMA" of
"Gaussian Mixture Attention: Linear-Time Sequence Mixing via Probabilistic
Latent Routing": the prefix memories and Eq. 8b, prefix j <= i inclusive).
It is tied to things other than itself: the oracle's causal forward, which
the C code computes as one sequential running sum; the bidirectional latent
memory of the whole sequence (the state the prefix reaches at i = N); the
closed-form running mean of the single-component case; and responsibilities
from scikit-learn's diagonal GMM.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle import _rand_problem, _sklearn_gamma


def _decode_all(Q, Kx, V, mu, ls2, alpha, eps):
    B, H, N, _ = Q.shape
    Kc, d_v = mu.shape[1], V.shape[-1]
    S = np.zeros((B, H, Kc, d_v))
    z = np.zeros((B, H, Kc))
    outs, aq, ak = [], [], []
    for i in range(N):
        r = oracle.decode_step(S, z, Q[:, :, i], Kx[:, :, i], V[:, :, i], mu, ls2, alpha, eps)
        S, z = r["S"], r["z"]
        outs.append(r["out"])
        aq.append(r["assign_q"])
        ak.append(r["assign_k"])
    return np.stack(outs, 2), np.stack(aq, 2), np.stack(ak, 2), S, z


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_from_empty_state_reproduces_causal_forward(seed):
    Q, Kx, V, mu, ls2, alpha = _rand_problem(seed, B=2, H=2, N=40, d_r=6, d_v=5, K=5)
    out, aq, ak, _, _ = _decode_all(Q, Kx, V, mu, ls2, alpha, 1e-6)
    ref = oracle.forward(Q, Kx, V, mu, ls2, alpha, 1e-6, True, want_assign=True)
    np.testing.assert_allclose(out, ref["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(aq, ref["assign_q"])
    np.testing.assert_array_equal(ak, ref["assign_k"])


def test_state_after_whole_sequence_is_the_latent_memory():
    Q, Kx, V, mu, ls2, alpha = _rand_problem(3, B=1, H=3, N=33, d_r=4, d_v=7, K=6)
    _, _, _, S, z = _decode_all(Q, Kx, V, mu, ls2, alpha, 1e-6)
    ref = oracle.forward(Q, Kx, V, mu, ls2, alpha, 1e-6, False, want_latent=True)
    np.testing.assert_allclose(S, ref["vtilde"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z, ref["z"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(z.sum(-1), 33.0, rtol=1e-12)


def test_single_component_decode_is_running_mean():
    Q, Kx, V, mu, ls2, alpha = _rand_problem(4, B=1, H=1, N=25, d_r=3, d_v=4, K=1)
    eps = 1e-3
    out, _, _, _, _ = _decode_all(Q, Kx, V, mu, ls2, alpha, eps)
    csum = np.cumsum(V, axis=2)
    count = np.arange(1, 26, dtype=np.float64)[None, None, :, None]
    np.testing.assert_allclose(out, csum / (count + eps), rtol=1e-12)


def test_decode_step_matches_sklearn_responsibilities():
    # an arbitrary non-negative state, one step, the update and read-out
    # written out with scikit-learn's posterior
    Q, Kx, V, mu, ls2, alpha = _rand_problem(5, B=2, H=2, N=1, d_r=5, d_v=3, K=4)
    rng = np.random.default_rng(6)
    S = rng.standard_normal((2, 2, 4, 3))
    z = rng.uniform(0.5, 3.0, (2, 2, 4))
    eps = 1e-6
    r = oracle.decode_step(S, z, Q[:, :, 0], Kx[:, :, 0], V[:, :, 0], mu, ls2, alpha, eps)
    gq = _sklearn_gamma(Q, mu, ls2, alpha)[:, :, 0]
    gk = _sklearn_gamma(Kx, mu, ls2, alpha)[:, :, 0]
    for b in range(2):
        for h in range(2):
            S2 = S[b, h] + np.outer(gk[b, h], V[b, h, 0])
            z2 = z[b, h] + gk[b, h]
            o = gq[b, h] @ S2 / (gq[b, h] @ z2 + eps)
            np.testing.assert_allclose(r["S"][b, h], S2, rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(r["z"][b, h], z2, rtol=1e-9)
            np.testing.assert_allclose(r["out"][b, h], o, rtol=1e-9, atol=1e-12)
