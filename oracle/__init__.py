"""CPU float64 oracle for streaming log-domain Sinkhorn (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; the product package never imports it. The
per-pair arithmetic lives in ``sk_oracle.c`` (plain float64 loops, OpenMP over
rows) and this file marshals numpy arrays to it; the composed references
(divergence, run to tolerance, dense Hessian-vector product and Newton step)
are written here in float64 numpy on top of those routines or from their
dense definitions, each with its derivation in its docstring.

Every function takes the stored point values exactly (float32, or bf16 decoded
exactly) promoted to float64, and weights as stored (float32) promoted to
float64. Conventions (see sk_oracle.c for the formulas and their sources):
  F(g)_i = -eps * LSE_j(log b_j + (g_j - C_ij)/eps), G symmetric,
  P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps), C_ij = |x_i - y_j|^2.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sk_oracle.c")
_LIB = os.path.join(_HERE, "libskoracle.so")

ALTERNATING, SYMMETRIC = 0, 1
_MODES = {"alternating": ALTERNATING, "symmetric": SYMMETRIC}

_lib = None


def build(force: bool = True) -> str:
    """Compile sk_oracle.c with gcc (IEEE float64: no fast-math) into libskoracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    INT = ctypes.c_int
    sig = {
        "sko_F": [P, P, I64, I64, I64, P, P, D, P],
        "sko_G": [P, P, I64, I64, I64, P, P, D, P],
        "sko_solve": [P, P, I64, I64, I64, P, P, D, INT, INT, P, P, P],
        "sko_grad_x": [P, P, I64, I64, I64, P, P, P, D, P],
        "sko_grad_x_plan": [P, P, I64, I64, I64, P, P, P, P, D, P],
        "sko_apply": [P, P, I64, I64, I64, P, P, P, P, D, INT, P, I64, P],
        "sko_apply_hadamard": [P, P, I64, I64, I64, P, P, P, P, D, INT, P, P, I64, P, I64, P],
        "sko_marginals": [P, P, I64, I64, I64, P, P, P, P, D, P, P],
        "sko_objectives": [P, P, I64, I64, I64, P, P, P, P, D, P, P],
        "sko_set_threads": [INT],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.sko_threads.restype = INT
    lib.sko_version.restype = INT
    _lib = lib
    return lib


def _c(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _shapes(x, y):
    x = _c(x)
    y = _c(y)
    if x.ndim == 1:
        x = x[:, None]
    if y.ndim == 1:
        y = y[:, None]
    assert x.shape[1] == y.shape[1], "x and y must have the same dimension"
    return x, y, x.shape[0], y.shape[0], x.shape[1]


def set_threads(t: int) -> None:
    _load().sko_set_threads(int(t))


def threads() -> int:
    return int(_load().sko_threads())


def F(x, y, b, g, eps):
    """F(g)_i = -eps * LSE_j(log b_j + (g_j - C_ij)/eps)."""
    x, y, n, m, d = _shapes(x, y)
    b, g = _c(b), _c(g)
    out = np.empty(n)
    _load().sko_F(_p(x), _p(y), n, m, d, _p(b), _p(g), float(eps), _p(out))
    return out


def G(x, y, a, f, eps):
    """G(f)_j = -eps * LSE_i(log a_i + (f_i - C_ij)/eps)."""
    x, y, n, m, d = _shapes(x, y)
    a, f = _c(a), _c(f)
    out = np.empty(m)
    _load().sko_G(_p(x), _p(y), n, m, d, _p(a), _p(f), float(eps), _p(out))
    return out


def solve(x, y, a, b, eps, iters, mode="alternating", f0=None, g0=None):
    """Fixed-budget Sinkhorn from (f0, g0) (zeros by default). Returns (f, g, cost)."""
    x, y, n, m, d = _shapes(x, y)
    a, b = _c(a), _c(b)
    f = np.zeros(n) if f0 is None else _c(f0).copy()
    g = np.zeros(m) if g0 is None else _c(g0).copy()
    cost = ctypes.c_double(0.0)
    _load().sko_solve(_p(x), _p(y), n, m, d, _p(a), _p(b), float(eps), int(iters),
                      _MODES[mode] if isinstance(mode, str) else int(mode),
                      _p(f), _p(g), ctypes.byref(cost))
    return f, g, cost.value


def grad_x(x, y, a, b, g, eps):
    """grad_i = 2 a_i (x_i - sum_j softmax_j(log b_j + (g_j - C_ij)/eps) y_j)."""
    x, y, n, m, d = _shapes(x, y)
    a, b, g = _c(a), _c(b), _c(g)
    out = np.empty((n, d))
    _load().sko_grad_x(_p(x), _p(y), n, m, d, _p(a), _p(b), _p(g), float(eps), _p(out))
    return out


def divergence(x, y, a, b, eps, iters, mode="alternating"):
    """Debiased Sinkhorn divergence and its gradients, composed from three solves.

    The FlashSinkhorn replication review names a "debiased-Sinkhorn" sweep
    among the OTDD drivers (Weaknesses, "Downstream drivers absent") without a
    formula; this is the textbook form
        S = OT(x,a; y,b) - OT(x,a; x,a)/2 - OT(y,b; y,b)/2,
    each OT the cost <a,f> + <b,g> of a fixed-budget solve: the cross term with
    `mode`, the two self terms with the symmetric schedule (which keeps f = g).
    Gradients (envelope argument at converged potentials; exact for the
    fixed-g maps at any iterate):
        d/da: f_ab - f_aa, d/db: g_ab - g_bb (each up to an additive constant
        when the weights are perturbed off the simplex);
        d/dx: grad_x(x; y, b, g_ab) - grad_x(x; x, a, g_aa)  (x enters the self
        term on both sides: twice the one-sided gradient, times 1/2);
        d/dy: grad_x(y; x, a, f_ab) - grad_x(y; y, b, g_bb).
    Returns (S, grad_a, grad_b, grad_x, grad_y).
    """
    f_ab, g_ab, c_ab = solve(x, y, a, b, eps, iters, mode)
    f_aa, g_aa, c_aa = solve(x, x, a, a, eps, iters, "symmetric")
    f_bb, g_bb, c_bb = solve(y, y, b, b, eps, iters, "symmetric")
    S = c_ab - 0.5 * c_aa - 0.5 * c_bb
    gx = grad_x(x, y, a, b, g_ab, eps) - grad_x(x, x, a, a, g_aa, eps)
    gy = grad_x(y, x, b, a, f_ab, eps) - grad_x(y, y, b, b, g_bb, eps)
    return S, f_ab - f_aa, g_ab - g_bb, gx, gy


def grad_x_plan(x, y, a, b, f, g, eps):
    """Diagnostic: 2 (r_i x_i - (P Y)_i) with P at (f, g)."""
    x, y, n, m, d = _shapes(x, y)
    a, b, f, g = _c(a), _c(b), _c(f), _c(g)
    out = np.empty((n, d))
    _load().sko_grad_x_plan(_p(x), _p(y), n, m, d, _p(a), _p(b), _p(f), _p(g), float(eps), _p(out))
    return out


def apply(x, y, a, b, f, g, eps, V, transpose=False):
    """P V (V: m x k) or, with transpose, P^T V (V: n x k)."""
    x, y, n, m, d = _shapes(x, y)
    a, b, f, g = _c(a), _c(b), _c(f), _c(g)
    V = _c(V)
    squeeze = V.ndim == 1
    if squeeze:
        V = V[:, None]
    k = V.shape[1]
    rows = m if transpose else n
    assert V.shape[0] == (n if transpose else m)
    out = np.empty((rows, k))
    _load().sko_apply(_p(x), _p(y), n, m, d, _p(a), _p(b), _p(f), _p(g), float(eps),
                      int(bool(transpose)), _p(V), k, _p(out))
    return out[:, 0] if squeeze else out


def apply_hadamard(x, y, a, b, f, g, eps, A, B, V, transpose=False):
    """(P o W) V (V: m x k) or, with transpose, (P o W)^T V (V: n x k), W = A B^T
    with A (n x r), B (m x r); evaluated entry by entry from the definition."""
    x, y, n, m, d = _shapes(x, y)
    a, b, f, g = _c(a), _c(b), _c(f), _c(g)
    A, B, V = _c(A), _c(B), _c(V)
    if A.ndim == 1:
        A = A[:, None]
    if B.ndim == 1:
        B = B[:, None]
    squeeze = V.ndim == 1
    if squeeze:
        V = V[:, None]
    r, k = A.shape[1], V.shape[1]
    assert A.shape == (n, r) and B.shape == (m, r) and V.shape[0] == (n if transpose else m)
    out = np.empty((m if transpose else n, k))
    _load().sko_apply_hadamard(_p(x), _p(y), n, m, d, _p(a), _p(b), _p(f), _p(g), float(eps),
                               int(bool(transpose)), _p(A), _p(B), r, _p(V), k, _p(out))
    return out[:, 0] if squeeze else out


def hvp_x(x, y, a, b, f, g, eps, V):
    """Hessian-vector product of OT_eps with respect to x, dense (small n, m).

    Implicit differentiation of the optimality conditions at the pair (f, g)
    (the review's Summary and Strengths describe the HVP as a Schur solve over
    streaming plan products, Theorem 5, checked against a dense Moore-Penrose
    reference; the pages print no formula, so it is derived here). With
    P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps), row and column sums r, c, and a
    tangent V (n x d) of x:
        dC_ij = 2 (x_i - y_j) . v_i
        u = (P o dC) 1,  w = (P o dC)^T 1
        [diag(r) P; P^T diag(c)] [df; dg] = [u; w]   (Moore-Penrose solution)
        dP_ij = P_ij (df_i + dg_j - dC_ij) / eps
        (H V)_i = 2 r_i v_i - 2 sum_j dP_ij y_j
    the derivative of the gradient 2 sum_j P_ij (x_i - y_j) with the marginals
    held fixed (sum_j dP_ij = 0 removes the x_i term). Returns n x d.
    """
    x, y = np.asarray(x, dtype=np.float64), np.asarray(y, dtype=np.float64)
    a, b, f, g = (np.asarray(t, dtype=np.float64) for t in (a, b, f, g))
    V = np.asarray(V, dtype=np.float64)
    diff = x[:, None, :] - y[None, :, :]
    C = (diff * diff).sum(-1)
    with np.errstate(divide="ignore"):
        P = np.exp(np.log(a)[:, None] + np.log(b)[None, :] + (f[:, None] + g[None, :] - C) / eps)
    r, c = P.sum(1), P.sum(0)
    dC = 2.0 * (diff * V[:, None, :]).sum(-1)
    u, w = (P * dC).sum(1), (P * dC).sum(0)
    n, m = P.shape
    K = np.zeros((n + m, n + m))
    K[:n, :n] = np.diag(r)
    K[:n, n:] = P
    K[n:, :n] = P.T
    K[n:, n:] = np.diag(c)
    sol = np.linalg.pinv(K) @ np.concatenate([u, w])
    df, dg = sol[:n], sol[n:]
    dP = P * (df[:, None] + dg[None, :] - dC) / eps
    return 2.0 * r[:, None] * V - 2.0 * dP @ y


def newton_x(x0, y, a, b, eps, newton_iters, sk_tol=1e-12, grad_tol=0.0, cg_max_iters=200, c1=1e-4,
             max_halvings=30):
    """Line-search Newton-CG on x -> OT_eps(mu_x, nu), mu_x = sum_i a_i delta_{x_i}.

    The replication review's Summary and Strengths present the streaming
    Hessian-vector product as what makes Newton-CG on OT_eps possible in
    O((n + m) d) memory; the pages print no algorithm, so the textbook
    line-search Newton-CG is used (inner CG truncated at the forcing term
    min(1/2, sqrt|g|) |g| or at the first direction of non-positive curvature,
    which falls back to -g on the first inner iteration; Armijo backtracking
    with c1 = 1e-4, halving up to max_halvings times, else stop). Every iterate
    solves Sinkhorn to the marginal error sk_tol (solve_tol, a check every 10
    iterations); the cost is <a, f> + <b, g>, the gradient grad_x (at converged
    potentials the gradient of OT_eps by the envelope argument) and H v hvp_x.
    Returns (x, costs, grad_norms, steps) over the iterates 0..steps.
    """
    x = np.array(x0, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    a, b = _c(a), _c(b)
    f, g, _, _ = solve_tol(x, y, a, b, eps, sk_tol, 10 ** 5, "alternating", 10)
    cost = float(a @ f + b @ g)
    costs, norms = [cost], []
    steps = 0
    for k in range(newton_iters + 1):
        grad = grad_x(x, y, a, b, g, eps)
        gn = float(np.sqrt((grad * grad).sum()))
        norms.append(gn)
        if k == newton_iters or gn <= grad_tol:
            break
        tolk = min(0.5, np.sqrt(gn)) * gn
        z = np.zeros_like(x)
        r = grad.copy()
        dv = -r
        rr = float((r * r).sum())
        p = None
        for j in range(cg_max_iters):
            Hd = hvp_x(x, y, a, b, f, g, eps, dv)
            curv = float((dv * Hd).sum())
            if curv <= 0.0:
                p = -grad if j == 0 else z
                break
            alpha = rr / curv
            z = z + alpha * dv
            r = r + alpha * Hd
            rr_new = float((r * r).sum())
            if np.sqrt(rr_new) < tolk:
                p = z
                break
            dv = -r + (rr_new / rr) * dv
            rr = rr_new
        if p is None:
            p = z
        slope = float((grad * p).sum())
        t = 1.0
        accepted = False
        for _ in range(max_halvings + 1):
            ft, gt, _, _ = solve_tol(x + t * p, y, a, b, eps, sk_tol, 10 ** 5, "alternating", 10)
            ct = float(a @ ft + b @ gt)
            if ct <= cost + c1 * t * slope:
                accepted = True
                break
            t *= 0.5
        if not accepted:
            break
        x = x + t * p
        f, g, cost = ft, gt, ct
        costs.append(cost)
        steps += 1
    return x, np.array(costs), np.array(norms), steps


def marginals(x, y, a, b, f, g, eps):
    """(P 1, P^T 1)."""
    x, y, n, m, d = _shapes(x, y)
    a, b, f, g = _c(a), _c(b), _c(f), _c(g)
    r = np.empty(n)
    c = np.empty(m)
    _load().sko_marginals(_p(x), _p(y), n, m, d, _p(a), _p(b), _p(f), _p(g), float(eps), _p(r), _p(c))
    return r, c


def objectives(x, y, a, b, f, g, eps):
    """(primal, dual) objective values at (f, g)."""
    x, y, n, m, d = _shapes(x, y)
    a, b, f, g = _c(a), _c(b), _c(f), _c(g)
    pr = ctypes.c_double()
    du = ctypes.c_double()
    _load().sko_objectives(_p(x), _p(y), n, m, d, _p(a), _p(b), _p(f), _p(g), float(eps),
                           ctypes.byref(pr), ctypes.byref(du))
    return pr.value, du.value


def solve_tol(x, y, a, b, eps, tol, max_iters, mode="alternating", check_every=10, eps_start=0.0):
    """Sinkhorn until the L1 marginal error ||P 1 - a||_1 + ||P^T 1 - b||_1 of a
    checked pair is <= tol, composed from solve() and marginals() (both in
    sk_oracle.c; the error is summed from the dense plan here, in float64).

    Schedule, as the library's tolerance solve states it: optional eps-scaling
    first (one iteration at each of eps_start, eps_start/2, ... while above
    eps); then iterations at eps, and after every check_every-th of them the
    pair before that iteration is checked (in the alternating schedule a pair
    not produced by an iteration at eps is skipped); the run stops after that
    iteration once the error is <= tol, or after max_iters iterations in all.
    Returns (f, g, iters_done, err) with err the last error measured (inf if none).
    """
    x, y, n, m, d = _shapes(x, y)
    a, b = _c(a), _c(b)
    f, g = np.zeros(n), np.zeros(m)
    done = 0
    ek = float(eps_start)
    while ek > eps and done < max_iters:
        f, g, _ = solve(x, y, a, b, ek, 1, mode, f, g)
        done += 1
        ek *= 0.5
    at_eps = 0
    err = float("inf")
    while done < max_iters:
        run = min(check_every - 1, max_iters - done - 1)
        if run > 0:
            f, g, _ = solve(x, y, a, b, eps, run, mode, f, g)
            done += run
            at_eps += run
        checked = (f.copy(), g.copy())
        measurable = mode == "symmetric" or at_eps > 0
        f, g, _ = solve(x, y, a, b, eps, 1, mode, f, g)
        done += 1
        at_eps += 1
        if not measurable:
            continue
        r, c = marginals(x, y, a, b, checked[0], checked[1], eps)
        err = float(np.abs(r - a).sum() + np.abs(c - b).sum())
        if err <= tol:
            break
    return f, g, done, err


def time_row_map(x, y, w, pot, eps, repeats: int = 1) -> float:
    """Wall seconds of one F-map evaluation (for the CPU-baseline timing)."""
    t0 = time.perf_counter()
    for _ in range(repeats):
        F(x, y, w, pot, eps)
    return (time.perf_counter() - t0) / repeats
