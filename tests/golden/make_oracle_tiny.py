"""Writes oracle_tiny.json: the oracle's outputs on small seeded inputs.

This is a regression fixture for the oracle itself (it guards against an
unintended change of its arithmetic); it calls only oracle/ and workloads/.
The pages print no worked example, so no stored value here comes from them.
Run from the repository root: python tests/golden/make_oracle_tiny.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

CASES = [(1, 40, 33, 6), (2, 37, 45, 5), (3, 24, 20, 4)]


def compute():
    out = []
    for key, n, m, iters in CASES:
        w = W.CASES[key].scaled(n, m, iters)
        inp = W.make_inputs(w)
        f, g, cost = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, iters, w.mode)
        grad = oracle.grad_x(inp.x64(), inp.y64(), inp.a, inp.b, g, w.eps)
        out.append({"config": key, "n": n, "m": m, "iters": iters, "eps": w.eps, "mode": w.mode,
                    "f": f.tolist(), "g": g.tolist(), "cost": cost, "grad_x": grad.ravel().tolist()})
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as fh:
        json.dump({"provenance": "tests/golden/make_oracle_tiny.py (oracle only)", "cases": compute()}, fh)
    print("wrote", path)
