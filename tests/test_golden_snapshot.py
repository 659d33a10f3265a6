"""The oracle still reproduces its committed snapshot (CPU only).

tests/golden/oracle_tiny_snapshot.json was written by tests/golden/make_golden.py,
which calls only the oracle. A change to the oracle's arithmetic that moves these
numbers must be justified by the pages or by a reading of them.
"""
import json
import os

import numpy as np

import oracle
from hla_inputs import WORKLOADS, layer_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_snapshot():
    with open(os.path.join(HERE, "golden", "oracle_tiny_snapshot.json")) as f:
        snap = json.load(f)
    w = WORKLOADS[0]
    assert snap["shape"] == [w.B, w.H, w.N, w.D]
    q, k, v, g = layer_inputs(w, 0)
    lin = oracle.gated_linear(q, k, v, g, snap["eps"])
    sm = oracle.gated_softmax(q, k, v, g, snap["scale"])
    rows = snap["rows"]
    np.testing.assert_allclose(lin[..., rows, :], np.array(snap["linear_rows"]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sm[..., rows, :], np.array(snap["softmax_rows"]), rtol=1e-12, atol=1e-14)
    assert abs(lin.sum() - snap["linear_sum"]) <= 1e-10 * max(1.0, abs(snap["linear_sum"]))
    assert abs((sm ** 2).sum() - snap["softmax_sumsq"]) <= 1e-10 * snap["softmax_sumsq"]
