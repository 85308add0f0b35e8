"""Writes oracle_newton.json: the float64 oracle's line-search Newton-CG on
the seeded cases of newton_cases.py (final points, costs and gradient norms
of every iterate), keyed by a digest of the oracle sources they depend on. It calls only
oracle/; no stored value comes from the GPU path.

    python tests/golden/make_oracle_newton.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

import newton_cases as NC  # noqa: E402
import oracle  # noqa: E402


def main():
    oracle.build(force=False)
    oracle.set_threads(1)  # tiny problems: one thread is fastest
    out = {"oracle_sha256": NC.oracle_digest(), "writer": "tests/golden/make_oracle_newton.py (oracle only)",
           "cases": []}
    for seed, n, m, d, eps in NC.CASES:
        x0, y, a, b = NC.inputs(seed, n, m, d)
        x, costs, norms, steps = oracle.newton_x(x0.astype(np.float64), y.astype(np.float64), a, b, eps,
                                                 NC.NEWTON_ITERS, sk_tol=1e-11, grad_tol=NC.GRAD_TOL)
        print(f"seed={seed} n={n} m={m} d={d} eps={eps}: {steps} steps, |grad| {norms[-1]:.2e}", flush=True)
        out["cases"].append({"seed": seed, "n": n, "m": m, "d": d, "eps": eps, "steps": steps,
                             "costs": costs.tolist(), "grad_norms": norms.tolist(), "x": x.ravel().tolist()})
    path = os.path.join(HERE, "oracle_newton.json")
    with open(path, "w") as fh:
        json.dump(out, fh)
    print("wrote", path)


if __name__ == "__main__":
    main()
