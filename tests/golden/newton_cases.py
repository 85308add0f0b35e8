"""Seeded inputs of the Newton-CG parity cases (float32 points), shared by the
writer of their stored oracle references and the GPU test. No arithmetic of
the method here: only draws and rounding."""
import numpy as np

# (seed, n, m, d, eps): register-resident records (d = 2) and GEMM-tiled ones
# (d = 32). Powers of two keep the float32 weights 1/n and 1/m exact, so both
# marginals hold the same mass and the float64 iteration can meet any tolerance.
CASES = [
    (5, 16, 32, 2, 0.1),
    (7, 32, 64, 2, 0.05),
    (3, 16, 32, 32, 0.5),
]
NEWTON_ITERS = 15
GRAD_TOL = 1e-5


def inputs(seed, n, m, d):
    rng = np.random.default_rng([seed, 77])
    y = rng.uniform(0, 1, (m, d)).astype(np.float32)
    x0 = rng.uniform(0, 1, (n, d)).astype(np.float32)
    if d > 2:
        y /= np.float32(np.sqrt(d))
        x0 /= np.float32(np.sqrt(d))
    a = np.full(n, np.float32(1.0 / n), dtype=np.float32)
    b = np.full(m, np.float32(1.0 / m), dtype=np.float32)
    return x0, y, a, b


def oracle_digest():
    """SHA-256 of what the stored Newton references depend on: the C oracle
    and the Python routines the float64 Newton-CG composes."""
    import hashlib
    import inspect
    import os

    import oracle
    h = hashlib.sha256()
    with open(os.path.join(os.path.dirname(oracle.__file__), "sk_oracle.c"), "rb") as fh:
        h.update(fh.read())
    for fn in (oracle.newton_x, oracle.solve_tol, oracle.hvp_x, oracle.grad_x, oracle.solve, oracle.marginals):
        h.update(inspect.getsource(fn).encode())
    return h.hexdigest()
