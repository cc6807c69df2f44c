"""Write tests/golden/tiny_*.txt from the fp64 oracle (calls only oracle/).

Workload: the tiny bidirectional fp32 case (B1 H1 N256 d_r16 d_v32 K8, seed 0)
in both variants; rows 0, 1, 127, 255 of the output and every hard assignment.
Regenerate with:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gaussian_mixture_sequence_gma_amd import inputs  # noqa: E402

ROWS = np.array([0, 1, 127, 255], dtype=np.int64)


def main():
    w = inputs.WORKLOADS["tiny_bidir_f32"]
    g = inputs.generate(w, 0)
    for causal in (False, True):
        r = oracle.forward(g["Q"].f32, g["K"].f32, g["V"].f32, g["mu"], g["log_sigma2"],
                           g["log_pi"], w.eps, causal, rows=ROWS, want_assign=True)
        full = oracle.forward(g["Q"].f32, g["K"].f32, g["V"].f32, g["mu"], g["log_sigma2"],
                              g["log_pi"], w.eps, causal, want_assign=True)
        name = "tiny_%s.txt" % ("causal" if causal else "bidir")
        with open(os.path.join(os.path.dirname(__file__), name), "w") as f:
            f.write("# fp64 oracle output, workload tiny_bidir_f32 seed 0, causal=%d\n" % causal)
            f.write("# written by tests/golden/make_golden.py\n")
            f.write("rows " + " ".join(str(int(x)) for x in ROWS) + "\n")
            for i, row in enumerate(r["out"][0, 0]):
                f.write("out %d " % ROWS[i] + " ".join("%.17e" % v for v in row) + "\n")
            f.write("assign_q " + " ".join(str(int(a)) for a in full["assign_q"][0, 0]) + "\n")
            f.write("assign_k " + " ".join(str(int(a)) for a in full["assign_k"][0, 0]) + "\n")


if __name__ == "__main__":
    main()
