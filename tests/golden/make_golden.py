"""Writes tests/golden/tiny_q4k_gemv.txt: the oracle's output on the tiny Q4_K
GEMV workload (N = K = 256, M = 1, fp32 activations, seed 0), together with
digests of its inputs. Calls only the oracle and the seeded input generator.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import qdm_synth  # noqa: E402


def main():
    w, x = qdm_synth.tiny_gemv()
    y = oracle.q4k_matmul(w, x, 256, 256)[0]
    lines = ["# oracle output, tiny Q4_K GEMV (N=K=256, M=1, fp32 x, seed 0)",
             "# written by tests/golden/make_golden.py (oracle + input generator only)",
             "w_sha256 " + hashlib.sha256(w.tobytes()).hexdigest(),
             "x_sha256 " + hashlib.sha256(x.tobytes()).hexdigest()]
    lines += ["y %d %s" % (n, float(v).hex()) for n, v in enumerate(y)]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_q4k_gemv.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
