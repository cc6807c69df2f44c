"""GPU parity of gma_usage_stats (component-usage diagnostics of the
responsibilities) against oracle.usage_stats.

Tolerances: mean responsibility and mean token entropy absolute 1e-4 (fp32
inputs) / 2e-3 (bf16: split-bf16 scores); counts and utilisations exact
except for tokens at a near-tie (argmax gap or |gamma - threshold| within
the assignment tie band of the parity tests), which may move; the usage
entropy and the number of components used must agree with the counts the
GPU reports (and with the oracle's when no token moved).
"""
import numpy as np
import pytest
import torch

import oracle
from gaussian_mixture_sequence_gma_amd import api, inputs
from tests.parity import TIE_DELTA, upload

pytestmark = pytest.mark.gpu

MEAN_TOL = {"f32": 1e-4, "bf16": 2e-3}


def _check(gen, X, dtype, thr, heads=None):
    dev = upload(gen)
    Xd = dev["Q"]
    got = api.usage_stats(Xd, dev["mu"], dev["log_sigma2"], dev["log_pi"], thr)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in got.items()}
    hs = slice(None) if heads is None else slice(0, heads)
    ref = oracle.usage_stats(X[:, hs], gen["mu"][hs], gen["log_sigma2"][hs], gen["log_pi"][hs],
                             thr)
    g = ref["gamma"]
    B, H, N, K = g.shape
    T = B * N
    # near-ties in the oracle's own arithmetic
    srt = np.sort(g, -1)
    sc = oracle.responsibilities(X[:, hs], gen["mu"][hs], gen["log_sigma2"][hs],
                                 gen["log_pi"][hs])["score"]
    ssrt = np.sort(sc, -1)
    tie = (ssrt[..., -1] - ssrt[..., -2] <= TIE_DELTA[dtype]) if K > 1 else np.zeros(g.shape[:3], bool)
    near_thr = np.abs(g - thr) <= MEAN_TOL[dtype]
    tol = MEAN_TOL[dtype]
    e_mean = np.abs(got["mean_gamma"][hs] - ref["mean_gamma"]).max()
    e_ent = np.abs(got["token_entropy"][hs] - ref["token_entropy"]).max()
    print("usage %s: mean_gamma %.2e  token_entropy %.2e  ties %d  near-threshold %d"
          % ((B, H, N, K, dtype), e_mean, e_ent, tie.sum(), near_thr.sum()))
    assert e_mean <= tol and e_ent <= tol
    for h in range(H):
        moved = np.abs(got["counts"][hs][h].astype(np.int64) - ref["counts"][h]).sum()
        assert moved <= 2 * tie[:, h].sum(), (h, moved)
        du = np.abs(got["utilization"][hs][h] - ref["utilization"][h]) * T
        assert (du <= near_thr[:, h].sum(axis=(0, 1)) + 1e-3).all(), h
        cnt = got["counts"][hs][h].astype(np.float64)
        p = cnt[cnt > 0] / T
        ue = -(p * np.log(p)).sum() / np.log(K) if K > 1 else 0.0
        assert abs(got["usage_entropy"][hs][h] - ue) <= 1e-5
        assert got["used"][hs][h] == np.count_nonzero(cnt)
        assert cnt.sum() == T
        if moved == 0:
            assert abs(got["usage_entropy"][hs][h] - ref["usage_entropy"][h]) <= 1e-5


@pytest.mark.parametrize("B,H,N,d_r,K,dtype,skew,thr", [
    (2, 3, 300, 32, 40, "f32", False, 0.1),
    (1, 2, 77, 16, 1, "f32", False, 0.1),
    (3, 2, 64, 64, 64, "f32", False, 0.0),
    (1, 4, 2000, 64, 128, "bf16", True, 0.1),
    (2, 2, 513, 128, 100, "bf16", False, 0.05),
    (1, 2, 700, 64, 256, "bf16", True, 0.1),   # K = 256 (the language-model setting)
    (2, 2, 300, 32, 200, "f32", False, 0.1),
])
def test_usage_stats_matches_oracle(B, H, N, d_r, K, dtype, skew, thr):
    kw = dict(mu_var=1.5, ls2_lo=-1.5, ls2_hi=0.5, logit_var=2.0) if skew else {}
    w = inputs.Workload("usage", B, H, N, d_r, 16, K, dtype, False, **kw)
    gen = inputs.generate(w, 21)
    _check(gen, gen["Q"].f32, dtype, thr)


def test_usage_stats_full_size_sampled_heads():
    """The long-context query tensor (B1 H32 N32768 d_r64 K128, bf16) in one
    launch; heads 0..3 checked against the oracle (heads are independent)."""
    w = inputs.WORKLOADS["long_bidir_bf16"]
    gen = inputs.generate(w, 0)
    _check(gen, gen["Q"].f32, "bf16", 0.1, heads=4)
