"""The tiny Q4_K GEMV workload: seeded inputs and the oracle's output on them
are stable (tests/golden/tiny_q4k_gemv.txt, written by make_golden.py)."""
import hashlib
import os

import numpy as np

import oracle
import qdm_synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_q4k_gemv.txt")


def load_golden():
    meta, y = {}, {}
    for line in open(GOLDEN):
        if line.startswith("#"):
            continue
        parts = line.split()
        if parts[0] == "y":
            y[int(parts[1])] = float.fromhex(parts[2])
        else:
            meta[parts[0]] = parts[1]
    return meta, np.array([y[i] for i in range(len(y))])


def test_tiny_inputs_and_oracle_output_stable():
    meta, y_gold = load_golden()
    w, x = qdm_synth.tiny_gemv()
    assert hashlib.sha256(w.tobytes()).hexdigest() == meta["w_sha256"]
    assert hashlib.sha256(x.tobytes()).hexdigest() == meta["x_sha256"]
    y = oracle.q4k_matmul(w, x, 256, 256)[0]
    np.testing.assert_array_equal(y, y_gold)
