"""Full-size oracle references: where they live and how they are keyed.

Each configuration's reference (``fullsize/<name>.npz``) holds the float64
oracle's results of the whole fixed-budget solve at the configuration's own
shape (every entry of f and g, and the cost), plus the gradient rows and
transport-application rows that configuration asks for. It is written once by
``make_oracle_fullsize.py`` (which calls only ``oracle/`` and ``workloads/``)
and keyed by two digests:
  * the input digest: SHA-256 of the stored bytes of x, y, a, b (and V, U when
    present) together with the workload's parameters, so a change of the
    generators makes the reference stale;
  * the oracle digest: SHA-256 of ``oracle/sk_oracle.c``, whose plain loops
    produced every stored number.
A test that finds either digest changed fails: the reference has to be
written again from the oracle.
"""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
DIR = os.path.join(HERE, "fullsize")
ORACLE_SRC = os.path.join(ROOT, "oracle", "sk_oracle.c")

# Configurations with a full-size reference, and the apply width of each.
KEYS = (2, 5, 4, 7, 3, 6)
SAMPLE_SEED = 20261203


def path_of(w) -> str:
    return os.path.join(DIR, w.name + ".npz")


def input_digest(inp) -> str:
    w = inp.w
    h = hashlib.sha256()
    h.update(json.dumps([w.cid, w.name, w.n, w.m, w.d, w.dtype, w.points, w.weights, w.eps, w.iters,
                         w.mode]).encode())
    for arr in (inp.x, inp.y, inp.a, inp.b, inp.V, inp.U):
        if arr is not None:
            h.update(np.ascontiguousarray(arr).tobytes())
    return h.hexdigest()


def oracle_digest() -> str:
    with open(ORACLE_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def sample(count: int, k: int, salt: int) -> np.ndarray:
    """Sorted sample of k distinct indices below count (all of them if k >= count)."""
    if k >= count:
        return np.arange(count)
    rng = np.random.default_rng([SAMPLE_SEED, salt])
    return np.sort(rng.choice(count, k, replace=False))


def load(w):
    """The stored reference of workload w as a dict, or None when absent."""
    p = path_of(w)
    if not os.path.exists(p):
        return None
    with np.load(p, allow_pickle=False) as z:
        ref = {k: z[k] for k in z.files}
    ref["meta"] = json.loads(str(ref["meta"]))
    return ref
