"""Writes the full-size oracle references (tests/golden/fullsize/<name>.npz).

For each configuration it runs the float64 CPU oracle over the whole
fixed-budget solve at the configuration's own shape, then the gradient rows
and transport-application rows the configuration asks for, and stores:
  f, g        every entry (float64), after the configuration's iterations
  cost        <a, f> + <b, g> at that pair
  grad_rows, grad          sampled rows of the barycentric gradient (final g)
  pv_rows, pv, pv_abs      sampled rows of P V and P |V| (oracle potentials)
  ptu_cols, ptu, ptu_abs   sampled columns of P^T U and P^T |U|
  meta        JSON: digests of the inputs and of the oracle source, timings
It calls only oracle/ and workloads/; no stored value comes from the GPU path.
Minutes to about an hour per configuration on 8 host threads.

    python tests/golden/make_oracle_fullsize.py [--keys 2,5,4,7,3,6] [--threads N]
"""
import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

import fullsize as FS  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402

GRAD_ROWS = 64      # sampled gradient rows (all rows when n * d is small)
APPLY_SAMPLE = 512  # sampled rows / columns of the applications


def make(key: int, log) -> str:
    w = W.CASES[key]
    inp = W.make_inputs(w)
    x64, y64 = inp.x64(), inp.y64()
    meta = {"config": key, "name": w.name, "n": w.n, "m": w.m, "d": w.d, "dtype": w.dtype, "eps": w.eps,
            "iters": w.iters, "mode": w.mode, "input_sha256": FS.input_digest(inp),
            "oracle_sha256": FS.oracle_digest(), "threads": oracle.threads(),
            "writer": "tests/golden/make_oracle_fullsize.py (oracle only)"}
    log(f"cfg {key} {w.name}: n={w.n} m={w.m} d={w.d} {w.dtype} eps={w.eps} {w.iters} {w.mode}")
    t0 = time.perf_counter()
    f, g, cost = oracle.solve(x64, y64, inp.a, inp.b, w.eps, w.iters, w.mode)
    meta["solve_s"] = time.perf_counter() - t0
    log(f"  solve {meta['solve_s']:.0f} s, cost {cost!r}")
    out = {"f": f, "g": g, "cost": np.float64(cost)}
    if w.grad:
        rows = FS.sample(w.n, w.n if w.n * w.d <= 200_000 else GRAD_ROWS, salt=1)
        t0 = time.perf_counter()
        out["grad_rows"] = rows
        out["grad"] = oracle.grad_x(x64[rows], y64, inp.a[rows], inp.b, g, w.eps)
        meta["grad_s"] = time.perf_counter() - t0
        log(f"  gradient rows {len(rows)}: {meta['grad_s']:.0f} s")
    if w.apply_k:
        t0 = time.perf_counter()
        rows = FS.sample(w.n, APPLY_SAMPLE, salt=2)
        cols = FS.sample(w.m, APPLY_SAMPLE, salt=3)
        out["pv_rows"] = rows
        out["pv"] = oracle.apply(x64[rows], y64, inp.a[rows], inp.b, f[rows], g, w.eps, inp.V)
        out["pv_abs"] = oracle.apply(x64[rows], y64, inp.a[rows], inp.b, f[rows], g, w.eps, np.abs(inp.V))
        out["ptu_cols"] = cols
        out["ptu"] = oracle.apply(x64, y64[cols], inp.a, inp.b[cols], f, g[cols], w.eps, inp.U, transpose=True)
        out["ptu_abs"] = oracle.apply(x64, y64[cols], inp.a, inp.b[cols], f, g[cols], w.eps, np.abs(inp.U),
                                      transpose=True)
        meta["apply_s"] = time.perf_counter() - t0
        log(f"  applications: {meta['apply_s']:.0f} s")
    os.makedirs(FS.DIR, exist_ok=True)
    path = FS.path_of(w)
    tmp = path + ".tmp.npz"
    np.savez(tmp, meta=np.array(json.dumps(meta)), **out)
    os.replace(tmp, path)
    log(f"  wrote {os.path.relpath(path, ROOT)}")
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--keys", default=",".join(str(k) for k in FS.KEYS))
    ap.add_argument("--threads", type=int, default=0)
    args = ap.parse_args()
    oracle.build(force=False)
    if args.threads:
        oracle.set_threads(args.threads)

    def log(msg):
        print(msg, flush=True)

    for key in (int(k) for k in args.keys.split(",")):
        make(key, log)


if __name__ == "__main__":
    main()
