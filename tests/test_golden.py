"""The oracle still reproduces its stored fixtures (regression, CPU only)."""
import os

import numpy as np
import pytest

import oracle
from gaussian_mixture_sequence_gma_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    rows, outs, aq, ak = None, [], None, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#"):
                continue
            tag, *vals = line.split()
            if tag == "rows":
                rows = np.array([int(v) for v in vals])
            elif tag == "out":
                outs.append([float(v) for v in vals[1:]])
            elif tag == "assign_q":
                aq = np.array([int(v) for v in vals])
            elif tag == "assign_k":
                ak = np.array([int(v) for v in vals])
    return rows, np.array(outs), aq, ak


@pytest.mark.parametrize("causal", [False, True])
def test_oracle_reproduces_golden(causal):
    rows, outs, aq, ak = load_golden("tiny_%s.txt" % ("causal" if causal else "bidir"))
    w = inputs.WORKLOADS["tiny_bidir_f32"]
    g = inputs.generate(w, 0)
    r = oracle.forward(g["Q"].f32, g["K"].f32, g["V"].f32, g["mu"], g["log_sigma2"],
                       g["log_pi"], w.eps, causal, want_assign=True)
    np.testing.assert_allclose(r["out"][0, 0, rows], outs, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(r["assign_q"][0, 0], aq)
    np.testing.assert_array_equal(r["assign_k"][0, 0], ak)
