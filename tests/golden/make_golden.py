"""Write tests/golden/tiny_f32_oracle.txt from the fp64 oracle.

The stored values come only from ``oracle`` applied to the seeded tiny-f32
workload (B=1, H=1, L=64, d_k=d_v=16, seed 0) of ``efla_workloads``.  The
fixture guards the oracle against silent drift; it is not a second opinion on
the method (the pin tests are).  Regenerate with:

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import efla_workloads  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(HERE, "tiny_f32_oracle.txt")


def main():
    w = efla_workloads.FORWARD_WORKLOADS["tiny-f32"]
    q, k, v, beta, S0 = efla_workloads.forward_inputs(w, seed=0)
    o, SL = oracle.forward(q, k, v, beta, S0)
    with open(OUT, "w") as f:
        f.write("# fp64 oracle outputs for workload tiny-f32, seed 0 (written by make_golden.py)\n")
        f.write("# section o: [64,16] row-major; section S_L: [16,16] row-major; %.17g\n")
        f.write("o\n")
        np.savetxt(f, o.reshape(64, 16), fmt="%.17g")
        f.write("S_L\n")
        np.savetxt(f, SL.reshape(16, 16), fmt="%.17g")
    print(OUT)


if __name__ == "__main__":
    main()
