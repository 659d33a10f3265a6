"""Writes tests/golden/oracle_tiny_snapshot.json from the fp64 oracle only.

A regression snapshot: the tiny fp32 workload (B=1, H=2, N=256, D=32, eps=1e-6,
scale=1/sqrt(32)), both operators, a few query rows per head plus whole-output
sums. Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from hla_inputs import WORKLOADS, layer_inputs  # noqa: E402

ROWS = [0, 1, 63, 128, 255]


def main():
    w = WORKLOADS[0]
    q, k, v, g = layer_inputs(w, 0)
    lin = oracle.gated_linear(q, k, v, g, w.eps)
    sm = oracle.gated_softmax(q, k, v, g, w.scale)
    snap = {
        "workload": w.name, "shape": [w.B, w.H, w.N, w.D], "eps": w.eps, "scale": w.scale,
        "rows": ROWS,
        "linear_rows": lin[..., ROWS, :].tolist(),
        "softmax_rows": sm[..., ROWS, :].tolist(),
        "linear_sum": float(lin.sum()), "linear_sumsq": float((lin ** 2).sum()),
        "softmax_sum": float(sm.sum()), "softmax_sumsq": float((sm ** 2).sum()),
    }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_snapshot.json")
    with open(out, "w") as f:
        json.dump(snap, f, indent=0)
    print("wrote", out)


if __name__ == "__main__":
    main()
