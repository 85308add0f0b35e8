"""Pins of the CPU float64 oracle against facts it does not compute itself.

Each test ties an oracle routine to an independent fact fixed by the pages or by
the mathematics of entropic optimal transport:
  * the primal matrix-scaling form of Sinkhorn (u = a / (K v), v = b / (K^T u)),
    derived in "Fused & Furious: Sinkhorn Triton Kernels", section II.B, with
    unit marginals there and general ones here;
  * marginal constraints and primal/dual agreement at convergence;
  * translation invariance and the swap symmetry of the averaged schedule;
  * closed forms (one point per side; two points per side with uniform weights);
  * the eps -> 0 limit against brute force over permutations, the extreme points
    of the Birkhoff polytope (same page, section II);
  * the eps-monotonicity and the product-coupling upper bound of OT_eps;
  * finite differences of the gradient, including the envelope (Danskin) argument
    named in the FlashSinkhorn replication review's Weaknesses paragraph;
  * the plan-rescaling identity of the block-wise Sinkhorn attention explainer,
    section 2.2 (plans at different potentials differ by diagonal scalings).
None of these tests uses a GPU.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.optimize import linprog

import oracle


def _cloud(seed, n, d, lo=0.0, hi=1.0):
    return np.random.default_rng([seed, 7]).uniform(lo, hi, size=(n, d))


def _weights(seed, n):
    w = np.random.default_rng([seed, 8]).exponential(1.0, size=n)
    return w / w.sum()


def _pairwise_by_expansion(x, y):
    """|x|^2 + |y|^2 - 2 x.y: a different evaluation from the oracle's differences."""
    return (x * x).sum(1)[:, None] + (y * y).sum(1)[None, :] - 2.0 * x @ y.T


def _scaling_iterates(K, a, b, iters, mode):
    """Primal matrix-scaling Sinkhorn from f = g = 0, i.e. u = a, v = b."""
    u, v = a.copy(), b.copy()
    for _ in range(iters):
        if mode == "alternating":
            u = a / (K @ v)
            v = b / (K.T @ u)
        else:  # averaged potentials <=> geometric mean of the scalings
            u, v = np.sqrt(u * a / (K @ v)), np.sqrt(v * b / (K.T @ u))
    return u, v


def _converge(x, y, a, b, eps, tol=1e-12, max_iters=200000):
    """Alternating oracle iterations until both marginals hold to tol."""
    f = np.zeros(len(a))
    g = np.zeros(len(b))
    done = 0
    step = 200
    while done < max_iters:
        f, g, cost = oracle.solve(x, y, a, b, eps, step, "alternating", f, g)
        done += step
        r, c = oracle.marginals(x, y, a, b, f, g, eps)
        if max(np.abs(r - a).max(), np.abs(c - b).max()) < tol:
            return f, g, cost
    raise AssertionError("no convergence")


# ---------------------------------------------------------------- P1 scaling form
@pytest.mark.parametrize("mode", ["alternating", "symmetric"])
def test_log_domain_matches_primal_scaling(mode):
    x, y = _cloud(1, 7, 3), _cloud(2, 5, 3)
    a, b = _weights(3, 7), _weights(4, 5) * 1.3  # unequal masses are allowed
    eps = 0.15
    K = np.exp(-_pairwise_by_expansion(x, y) / eps)
    for iters in (1, 2, 5, 17):
        u, v = _scaling_iterates(K, a, b, iters, mode)
        f, g, _ = oracle.solve(x, y, a, b, eps, iters, mode)
        np.testing.assert_allclose(f, eps * np.log(u / a), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g, eps * np.log(v / b), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P2 marginals
def test_half_step_marginals_are_exact():
    x, y = _cloud(5, 9, 2), _cloud(6, 11, 2)
    a, b = _weights(7, 9), _weights(8, 11)
    eps = 0.2
    f, g, _ = oracle.solve(x, y, a, b, eps, 3, "alternating")
    r, c = oracle.marginals(x, y, a, b, f, g, eps)
    np.testing.assert_allclose(c, b, rtol=1e-13)          # g = G(f) makes P^T 1 = b
    f2 = oracle.F(x, y, b, g, eps)
    r2, _ = oracle.marginals(x, y, a, b, f2, g, eps)
    np.testing.assert_allclose(r2, a, rtol=1e-13)         # f = F(g) makes P 1 = a


def test_marginals_at_convergence_and_primal_equals_dual():
    x, y = _cloud(9, 8, 3), _cloud(10, 6, 3)
    a, b = _weights(11, 8), _weights(12, 6)
    eps = 0.1
    f, g, cost = _converge(x, y, a, b, eps, tol=1e-12)
    r, c = oracle.marginals(x, y, a, b, f, g, eps)
    assert np.abs(r - a).max() < 1e-10 and np.abs(c - b).max() < 1e-10
    primal, dual = oracle.objectives(x, y, a, b, f, g, eps)
    assert abs(primal - dual) <= 1e-10 * abs(primal)
    assert abs(cost - dual) <= 1e-10 * abs(primal)


def test_cost_equals_full_dual_after_each_alternating_iteration():
    x, y = _cloud(13, 6, 2), _cloud(14, 7, 2)
    a, b = _weights(15, 6), _weights(16, 7)
    eps = 0.3
    for iters in (1, 2, 4):
        f, g, cost = oracle.solve(x, y, a, b, eps, iters)
        _, dual = oracle.objectives(x, y, a, b, f, g, eps)
        assert abs(cost - dual) < 1e-13 * max(1.0, abs(cost))


# ---------------------------------------------------------------- P4 / P5 invariances
def test_translation_invariance():
    x, y = _cloud(17, 10, 3), _cloud(18, 12, 3)
    a, b = _weights(19, 10), _weights(20, 12)
    eps = 0.05
    t = np.array([0.3, -1.7, 2.2])
    f1, g1, c1 = oracle.solve(x, y, a, b, eps, 30)
    f2, g2, c2 = oracle.solve(x + t, y + t, a, b, eps, 30)
    np.testing.assert_allclose(f2, f1, atol=1e-11)
    np.testing.assert_allclose(g2, g1, atol=1e-11)
    assert abs(c2 - c1) < 1e-11
    gr1 = oracle.grad_x(x, y, a, b, g1, eps)
    gr2 = oracle.grad_x(x + t, y + t, a, b, g2, eps)
    np.testing.assert_allclose(gr2, gr1, atol=1e-9)


def test_symmetric_schedule_is_swap_symmetric():
    x, y = _cloud(21, 9, 2), _cloud(22, 6, 2)
    a, b = _weights(23, 9), _weights(24, 6)
    eps = 0.1
    f, g, c = oracle.solve(x, y, a, b, eps, 13, "symmetric")
    f_s, g_s, c_s = oracle.solve(y, x, b, a, eps, 13, "symmetric")
    assert np.array_equal(f_s, g) and np.array_equal(g_s, f)
    assert abs(c_s - c) < 1e-14
    # the alternating schedule is not symmetric: this guards the test itself
    fa, ga, _ = oracle.solve(x, y, a, b, eps, 3, "alternating")
    fb, gb, _ = oracle.solve(y, x, b, a, eps, 3, "alternating")
    assert not np.allclose(fb, ga)


# ---------------------------------------------------------------- P6 closed forms
def test_single_point_each_side():
    x = np.array([[0.0, 0.0]])
    y = np.array([[3.0, 4.0]])          # C = 25
    one = np.ones(1)
    eps = 0.7
    f, g, cost = oracle.solve(x, y, one, one, eps, 1, "alternating")
    assert f[0] == pytest.approx(25.0, abs=1e-12) and g[0] == pytest.approx(0.0, abs=1e-12)
    assert cost == pytest.approx(25.0, abs=1e-12)
    f, g, cost = oracle.solve(x, y, one, one, eps, 1, "symmetric")
    assert f[0] == pytest.approx(12.5, abs=1e-12) and g[0] == pytest.approx(12.5, abs=1e-12)
    # unit weights other than 1: F(0) = C - eps log b
    f, g, _ = oracle.solve(x, y, np.array([2.0]), np.array([0.5]), eps, 1, "alternating")
    assert f[0] == pytest.approx(25.0 - eps * math.log(0.5), abs=1e-12)
    # then G(f) = C - eps log a - f, so f + g = C - eps log a
    assert f[0] + g[0] == pytest.approx(25.0 - eps * math.log(2.0), abs=1e-12)


def test_two_by_two_closed_form_plan_and_cost():
    # Uniform 2x2: the optimal plan is [[p, 1/2-p], [1/2-p, p]] with
    # p / (1/2 - p) = exp(-(C11 + C22 - C12 - C21) / (2 eps)).
    x = np.array([[0.0, 0.0], [1.0, 0.5]])
    y = np.array([[0.2, 0.1], [0.7, 0.9]])
    C = _pairwise_by_expansion(x, y)
    a = b = np.array([0.5, 0.5])
    for eps in (0.15, 0.3, 2.0):
        kappa = math.exp(-(C[0, 0] + C[1, 1] - C[0, 1] - C[1, 0]) / (2 * eps))
        p = kappa / (2 * (1 + kappa))
        P = np.array([[p, 0.5 - p], [0.5 - p, p]])
        ot = (P * C).sum() + eps * (P * np.log(P / 0.25)).sum()
        f, g, cost = _converge(x, y, a, b, eps, tol=1e-14 if eps > 0.2 else 1e-13)
        assert cost == pytest.approx(ot, rel=1e-11, abs=1e-13)
        cols = oracle.apply(x, y, a, b, f, g, eps, np.eye(2))   # P @ I
        np.testing.assert_allclose(cols, P, rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------- P7 / P8 eps limits
def _lp_ot(C, a, b):
    n, m = C.shape
    A_eq = np.zeros((n + m, n * m))
    for i in range(n):
        A_eq[i, i * m:(i + 1) * m] = 1.0
    for j in range(m):
        A_eq[n + j, j::m] = 1.0
    res = linprog(C.ravel(), A_eq=A_eq, b_eq=np.concatenate([a, b]), bounds=(0, None), method="highs")
    assert res.status == 0
    return res.fun


def test_eps_monotone_and_bounded_by_product_coupling():
    x, y = _cloud(31, 6, 2), _cloud(32, 5, 2)
    a, b = _weights(33, 6), _weights(34, 5)
    C = _pairwise_by_expansion(x, y)
    ot0 = _lp_ot(C, a, b)
    # <a (x) b, C> = sum a|x|^2 + sum b|y|^2 - 2 <sum a x, sum b y> for unit masses
    prod = a @ (x * x).sum(1) + b @ (y * y).sum(1) - 2.0 * (a @ x) @ (b @ y)
    prev = -np.inf
    for eps in (0.05, 0.1, 0.3, 1.0, 3.0):
        _, _, c = _converge(x, y, a, b, eps, tol=1e-11)
        assert ot0 - 1e-9 <= c <= prod + 1e-12
        assert c >= prev - 1e-12
        prev = c
    _, _, c_big = _converge(x, y, a, b, 1e4, tol=1e-13)
    assert c_big == pytest.approx(prod, rel=1e-4)


@pytest.mark.parametrize("n", [4, 6])
def test_small_eps_against_brute_force_permutations(n):
    x, y = _cloud(40 + n, n, 2), _cloud(50 + n, n, 2)
    a = b = np.full(n, 1.0 / n)
    C = _pairwise_by_expansion(x, y)
    ot0 = min(sum(C[i, s[i]] for i in range(n)) for s in itertools.permutations(range(n))) / n
    for eps in (0.02, 0.05, 0.2):
        _, _, c = _converge(x, y, a, b, eps, tol=1e-11)
        # a permutation plan divided by n has KL(P | a (x) b) = log n
        assert ot0 - 1e-9 <= c <= ot0 + eps * math.log(n) + 1e-9


# ---------------------------------------------------------------- P9 gradient
def test_gradient_matches_finite_differences_at_fixed_g():
    x, y = _cloud(61, 5, 3), _cloud(62, 7, 3)
    a, b = _weights(63, 5), _weights(64, 7)
    eps = 0.2
    _, g, _ = oracle.solve(x, y, a, b, eps, 4)           # any iterate will do
    grad = oracle.grad_x(x, y, a, b, g, eps)

    def obj(xx):
        return a @ oracle.F(xx, y, b, g, eps) + b @ g

    h = 1e-5
    fd = np.zeros_like(x)
    for i in range(x.shape[0]):
        for k in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[i, k] += h
            xm[i, k] -= h
            fd[i, k] = (obj(xp) - obj(xm)) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-9)


def test_gradient_envelope_at_convergence_and_plan_form():
    x, y = _cloud(65, 4, 2), _cloud(66, 5, 2)
    a, b = _weights(67, 4), _weights(68, 5)
    eps = 0.25
    f, g, _ = _converge(x, y, a, b, eps, tol=1e-13)
    grad = oracle.grad_x(x, y, a, b, g, eps)
    h = 1e-5
    for i, k in [(0, 0), (2, 1), (3, 0)]:
        xp, xm = x.copy(), x.copy()
        xp[i, k] += h
        xm[i, k] -= h
        cp = _converge(xp, y, a, b, eps, tol=1e-13)[2]
        cm = _converge(xm, y, a, b, eps, tol=1e-13)[2]
        assert (cp - cm) / (2 * h) == pytest.approx(grad[i, k], rel=1e-5, abs=1e-8)
    # with f = F(g) the plan form 2 (r_i x_i - (P y)_i) equals the normalized form
    f_exact = oracle.F(x, y, b, g, eps)
    np.testing.assert_allclose(oracle.grad_x_plan(x, y, a, b, f_exact, g, eps), grad, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- P10 apply
def test_apply_identities():
    x, y = _cloud(71, 9, 3), _cloud(72, 8, 3)
    a, b = _weights(73, 9), _weights(74, 8)
    eps = 0.15
    rng = np.random.default_rng(75)
    f, g = rng.standard_normal(9) * 0.1, rng.standard_normal(8) * 0.1
    V, U = rng.standard_normal((8, 4)), rng.standard_normal((9, 4))
    PV = oracle.apply(x, y, a, b, f, g, eps, V)
    PtU = oracle.apply(x, y, a, b, f, g, eps, U, transpose=True)
    # adjointness <U, P V> = <P^T U, V>
    assert (U * PV).sum() == pytest.approx((PtU * V).sum(), rel=1e-12)
    # linearity in V
    np.testing.assert_allclose(oracle.apply(x, y, a, b, f, g, eps, 2.0 * V - U[:8]),
                               2.0 * PV - oracle.apply(x, y, a, b, f, g, eps, U[:8]), rtol=1e-11, atol=1e-14)
    # rescaling: P(f + delta, g) = diag(exp(delta/eps)) P(f, g)
    delta = rng.standard_normal(9) * 0.05
    np.testing.assert_allclose(oracle.apply(x, y, a, b, f + delta, g, eps, V),
                               np.exp(delta / eps)[:, None] * PV, rtol=1e-11)
    # after f = F(g) the row sums are exactly a; after g = G(f) the column sums are b
    f1 = oracle.F(x, y, b, g, eps)
    np.testing.assert_allclose(oracle.apply(x, y, a, b, f1, g, eps, np.ones(8)), a, rtol=1e-13)
    g1 = oracle.G(x, y, a, f, eps)
    np.testing.assert_allclose(oracle.apply(x, y, a, b, f, g1, eps, np.ones(9), transpose=True), b, rtol=1e-13)


# ---------------------------------------------------------------- maps: gauge and contraction
def test_map_gauge_and_nonexpansive():
    x, y = _cloud(81, 10, 2), _cloud(82, 12, 2)
    a, b = _weights(83, 10), _weights(84, 12)
    eps = 0.1
    rng = np.random.default_rng(85)
    g1, g2 = rng.standard_normal(12), rng.standard_normal(12)
    F1, F2 = oracle.F(x, y, b, g1, eps), oracle.F(x, y, b, g2, eps)
    np.testing.assert_allclose(oracle.F(x, y, b, g1 + 0.37, eps), F1 - 0.37, rtol=1e-13, atol=1e-13)

    def osc(v):
        return v.max() - v.min()
    # the log-domain map is an average (softmin), so it cannot expand oscillations
    assert osc(F1 - F2) <= osc(g1 - g2) + 1e-13
    assert np.all(F1 - F2 <= (g2 - g1).max() + 1e-13) and np.all(F1 - F2 >= (g2 - g1).min() - 1e-13)


def test_zero_weights_drop_out():
    x, y = _cloud(91, 6, 2), _cloud(92, 7, 2)
    a, b = _weights(93, 6), _weights(94, 7)
    b0 = b.copy()
    b0[[1, 4]] = 0.0
    eps = 0.2
    f, g, cost = oracle.solve(x, y, a, b0, eps, 5)
    keep = [0, 2, 3, 5, 6]
    fk, gk, ck = oracle.solve(x, y[keep], a, b0[keep], eps, 5)
    np.testing.assert_allclose(f, fk, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[keep], gk, rtol=1e-12, atol=1e-14)
    assert cost == pytest.approx(ck, rel=1e-12)


# ---------------------------------------------------------------- debiased divergence
# The review names a "debiased-Sinkhorn" sweep (Weaknesses, "Downstream drivers
# absent"); S = OT(a,b) - OT(a,a)/2 - OT(b,b)/2 is the textbook form. Its pins:
# it vanishes on identical inputs, is positive otherwise (the kernel
# exp(-|x-y|^2/eps) is positive definite), is symmetric under swapping the two
# measures, and its gradients match central differences of S itself.
_DIV_ITERS = 3000


def test_divergence_vanishes_on_identical_inputs_and_is_positive():
    eps = 0.1
    x, a = _cloud(101, 7, 2), _weights(102, 7)
    assert abs(oracle.divergence(x, x, a, a, eps, _DIV_ITERS)[0]) < 1e-12
    for seed in range(3):
        y, b = _cloud(110 + seed, 6 + seed, 2, 0.2, 1.3), _weights(120 + seed, 6 + seed)
        assert oracle.divergence(x, y, a, b, eps, _DIV_ITERS)[0] > 1e-4


def test_divergence_is_swap_symmetric():
    eps = 0.15
    x, y = _cloud(131, 6, 3), _cloud(132, 8, 3, 0.1, 1.1)
    a, b = _weights(133, 6), _weights(134, 8)
    s1 = oracle.divergence(x, y, a, b, eps, _DIV_ITERS)[0]
    s2 = oracle.divergence(y, x, b, a, eps, _DIV_ITERS)[0]
    assert s1 == pytest.approx(s2, rel=1e-10)


def test_divergence_gradients_match_finite_differences():
    eps, h = 0.1, 1e-6
    x, y = _cloud(141, 6, 2), _cloud(142, 7, 2, 0.2, 1.2)
    a, b = _weights(143, 6), _weights(144, 7)

    def S(x_, y_, a_, b_):
        return oracle.divergence(x_, y_, a_, b_, eps, _DIV_ITERS)[0]

    _, ga, gb, gx, gy = oracle.divergence(x, y, a, b, eps, _DIV_ITERS)
    for (i, k) in [(0, 0), (3, 1), (5, 0)]:
        xp, xm = x.copy(), x.copy()
        xp[i, k] += h
        xm[i, k] -= h
        assert (S(xp, y, a, b) - S(xm, y, a, b)) / (2 * h) == pytest.approx(gx[i, k], rel=1e-6, abs=1e-8)
    for (j, k) in [(1, 1), (6, 0)]:
        yp, ym = y.copy(), y.copy()
        yp[j, k] += h
        ym[j, k] -= h
        assert (S(x, yp, a, b) - S(x, ym, a, b)) / (2 * h) == pytest.approx(gy[j, k], rel=1e-6, abs=1e-8)
    # weights: directions that keep the total mass (the gradients are defined
    # up to an additive constant off the simplex)
    da = np.zeros(6)
    da[[1, 4]] = [1.0, -1.0]
    db = np.zeros(7)
    db[[0, 5]] = [1.0, -1.0]
    assert (S(x, y, a + h * da, b) - S(x, y, a - h * da, b)) / (2 * h) == pytest.approx(ga @ da, rel=1e-6)
    assert (S(x, y, a, b + h * db) - S(x, y, a, b - h * db)) / (2 * h) == pytest.approx(gb @ db, rel=1e-6)


# ---------------------------------------------------------------- Hadamard-weighted transport
# (P o W) V with W = A B^T (the review's Summary item ii names Hadamard-weighted
# applications; W is not defined on the pages). Pins against the plain
# application, which shares no code with it: W = 1 gives P V; a rank-one W =
# u v^T gives diag(u) P diag(v) V; the result is linear in W (sum of ranks).
def test_hadamard_apply_special_cases():
    x, y = _cloud(151, 7, 3), _cloud(152, 9, 3)
    a, b = _weights(153, 7), _weights(154, 9)
    rng = np.random.default_rng(155)
    f, g = rng.standard_normal(7) * 0.1, rng.standard_normal(9) * 0.1
    eps = 0.3
    V, U = rng.standard_normal((9, 4)), rng.standard_normal((7, 4))
    ones_n, ones_m = np.ones((7, 1)), np.ones((9, 1))
    np.testing.assert_allclose(oracle.apply_hadamard(x, y, a, b, f, g, eps, ones_n, ones_m, V),
                               oracle.apply(x, y, a, b, f, g, eps, V), rtol=1e-13)
    u, v = rng.standard_normal(7), rng.standard_normal(9)
    ref = u[:, None] * oracle.apply(x, y, a, b, f, g, eps, v[:, None] * V)
    np.testing.assert_allclose(oracle.apply_hadamard(x, y, a, b, f, g, eps, u, v, V), ref, rtol=1e-12, atol=1e-15)
    reft = v[:, None] * oracle.apply(x, y, a, b, f, g, eps, u[:, None] * U, transpose=True)
    np.testing.assert_allclose(oracle.apply_hadamard(x, y, a, b, f, g, eps, u, v, U, transpose=True), reft,
                               rtol=1e-12, atol=1e-15)
    A, B = rng.standard_normal((7, 3)), rng.standard_normal((9, 3))
    parts = sum(oracle.apply_hadamard(x, y, a, b, f, g, eps, A[:, s], B[:, s], V) for s in range(3))
    np.testing.assert_allclose(oracle.apply_hadamard(x, y, a, b, f, g, eps, A, B, V), parts, rtol=1e-12,
                               atol=1e-15)


# ---------------------------------------------------------------- Hessian-vector product
# The HVP of OT_eps in x (review, Summary and Strengths: Theorem 5's Schur solve
# over streaming plan products, checked against a dense Moore-Penrose
# reference). Pins: central differences of the converged gradient, and the
# symmetry of the Hessian.
def test_hvp_matches_finite_differences_of_the_converged_gradient():
    x, y = _cloud(161, 6, 2), _cloud(162, 7, 2, 0.2, 1.2)
    a, b = _weights(163, 6), _weights(164, 7)
    eps, h = 0.1, 1e-5
    f, g, _ = _converge(x, y, a, b, eps)
    V = np.random.default_rng(165).standard_normal((6, 2))

    def grad(xx):
        _, gg, _ = _converge(xx, y, a, b, eps)
        return oracle.grad_x(xx, y, a, b, gg, eps)
    fd = (grad(x + h * V) - grad(x - h * V)) / (2 * h)
    H = oracle.hvp_x(x, y, a, b, f, g, eps, V)
    assert np.abs(fd - H).max() <= 1e-7 * np.abs(H).max()


def test_hvp_is_symmetric():
    x, y = _cloud(171, 5, 3), _cloud(172, 8, 3, 0.1, 1.1)
    a, b = _weights(173, 5), _weights(174, 8)
    eps = 0.2
    f, g, _ = _converge(x, y, a, b, eps)
    rng = np.random.default_rng(175)
    U, V = rng.standard_normal((5, 3)), rng.standard_normal((5, 3))
    lhs = (U * oracle.hvp_x(x, y, a, b, f, g, eps, V)).sum()
    rhs = (V * oracle.hvp_x(x, y, a, b, f, g, eps, U)).sum()
    assert lhs == pytest.approx(rhs, rel=1e-10)


# ---------------------------------------------------------------- run to tolerance
def _scaling_solve_tol(K, a, b, tol, max_iters, check_every, mode):
    """The stopping rule of the tolerance solve on primal matrix scaling
    (u = a / (K v), v = b / (K^T u); P = diag(u) K diag(v)): after every
    check_every-th iteration, the marginal error of the pair before it."""
    u, v = a.copy(), b.copy()
    done = 0
    err = float("inf")
    while done < max_iters:
        run = min(check_every - 1, max_iters - done - 1)
        for _ in range(run):
            u, v = _scaling_iterates_from(K, a, b, u, v, mode)
        done += run
        uc, vc = u.copy(), v.copy()
        u, v = _scaling_iterates_from(K, a, b, u, v, mode)
        done += 1
        if mode == "alternating" and done == 1:
            continue
        P = uc[:, None] * K * vc[None, :]
        err = np.abs(P.sum(1) - a).sum() + np.abs(P.sum(0) - b).sum()
        if err <= tol:
            break
    return u, v, done, err


def _scaling_iterates_from(K, a, b, u, v, mode):
    if mode == "alternating":
        u = a / (K @ v)
        return u, b / (K.T @ u)
    return np.sqrt(u * a / (K @ v)), np.sqrt(v * b / (K.T @ u))


@pytest.mark.parametrize("mode,eps,tol,every", [("alternating", 0.05, 1e-6, 10), ("symmetric", 0.05, 1e-5, 7),
                                                ("alternating", 0.02, 1e-8, 1), ("alternating", 0.1, 1e-3, 4)])
def test_solve_tol_matches_primal_scaling_with_the_same_stopping_rule(mode, eps, tol, every):
    """The oracle's run to tolerance stops at the same iteration as primal matrix
    scaling under the same rule, with the same pair and error (the scaling form
    of the iteration: Fused & Furious, section II.B)."""
    x, y = _cloud(31, 9, 2), _cloud(32, 11, 2)
    a, b = _weights(33, 9), _weights(34, 11)
    K = np.exp(-_pairwise_by_expansion(x, y) / eps)
    u, v, n_s, e_s = _scaling_solve_tol(K, a, b, tol, 5000, every, mode)
    f, g, n_o, e_o = oracle.solve_tol(x, y, a, b, eps, tol, 5000, mode, every)
    assert n_o == n_s < 5000
    assert e_o == pytest.approx(e_s, rel=1e-6, abs=1e-14) and e_o <= tol
    np.testing.assert_allclose(np.exp(f / eps), u / a, rtol=1e-9)
    np.testing.assert_allclose(np.exp(g / eps), v / b, rtol=1e-9)


def test_solve_tol_eps_scaling_schedule():
    """eps-scaling runs one iteration per halving above eps before the checks:
    from eps_start = 0.8 to eps = 0.1 that is 0.8, 0.4, 0.2 (three iterations),
    whose pair then starts the run at eps."""
    x, y = _cloud(41, 8, 3), _cloud(42, 10, 3)
    a, b = _weights(43, 8), _weights(44, 10)
    f3, g3, _ = oracle.solve(x, y, a, b, 0.8, 1)
    f3, g3, _ = oracle.solve(x, y, a, b, 0.4, 1, "alternating", f3, g3)
    f3, g3, _ = oracle.solve(x, y, a, b, 0.2, 1, "alternating", f3, g3)
    fr, gr, _ = oracle.solve(x, y, a, b, 0.1, 20, "alternating", f3, g3)
    f, g, done, err = oracle.solve_tol(x, y, a, b, 0.1, 0.0, 23, "alternating", 10, eps_start=0.8)
    assert done == 23 and np.isfinite(err)
    np.testing.assert_allclose(f, fr, rtol=0, atol=1e-13)
    np.testing.assert_allclose(g, gr, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- Newton-CG
def _newton_instance(seed=5, n=10, m=24, d=2):
    rng = np.random.default_rng(seed)
    y = rng.uniform(0, 1, (m, d))
    x0 = rng.uniform(0, 1, (n, d))
    return x0, y, np.full(n, 1.0 / n), np.full(m, 1.0 / m)


def test_newton_reaches_a_stationary_point_with_decreasing_cost():
    """Line-search Newton-CG on x -> OT_eps(mu_x, nu): the costs decrease
    (Armijo), the gradient norm falls below 1e-8, the last steps converge
    superlinearly, and the limit is a fixed point of the barycentric map,
    r_i x_i = (P Y)_i, checked with the plan's own row sums and application
    (not with the gradient routine)."""
    x0, y, a, b = _newton_instance()
    eps = 0.1
    x, costs, norms, steps = oracle.newton_x(x0, y, a, b, eps, 12, sk_tol=1e-13, grad_tol=1e-9)
    assert np.all(np.diff(costs) < 1e-15)
    assert norms[-1] < 1e-8 and steps < 12
    tail = norms[-4:]  # the full Newton steps at the end
    # superlinear there: |g_{k+1}| <= e |g_k|^1.3
    assert all(np.log(tail[i + 1]) <= 1.3 * np.log(tail[i]) + 1.0 for i in range(len(tail) - 1))
    f, g, _, _ = oracle.solve_tol(x, y, a, b, eps, 1e-13, 10 ** 7, "alternating", 10)
    r, _ = oracle.marginals(x, y, a, b, f, g, eps)
    PY = oracle.apply(x, y, a, b, f, g, eps, y)
    assert np.abs(r[:, None] * x - PY).max() < 1e-9


def test_newton_step_solves_the_newton_system_by_finite_differences():
    """Near the minimizer the first inner CG direction p satisfies H p = -grad,
    H p taken here as a central difference of the converged gradient (not the
    Hessian-vector routine the step uses)."""
    x0, y, a, b = _newton_instance()
    eps = 0.1
    xs, _, _, _ = oracle.newton_x(x0, y, a, b, eps, 12, sk_tol=1e-13, grad_tol=1e-9)
    xk = xs + 0.01 * np.random.default_rng(9).standard_normal(xs.shape)

    def conv_grad(xx):
        f, g, _, _ = oracle.solve_tol(xx, y, a, b, eps, 1e-14, 10 ** 7, "alternating", 10)
        return oracle.grad_x(xx, y, a, b, g, eps)
    g0 = conv_grad(xk)
    x1, _, _, steps = oracle.newton_x(xk, y, a, b, eps, 1, sk_tol=1e-13)
    assert steps == 1
    p = x1 - xk  # the full step (t = 1 near the minimizer)
    h = 1e-4
    Hp = (conv_grad(xk + h * p) - conv_grad(xk - h * p)) / (2 * h)
    # the inner CG stops at the forcing term min(1/2, sqrt|g|) |g|
    gn = np.linalg.norm(g0)
    assert np.linalg.norm(Hp + g0) <= 1.05 * min(0.5, np.sqrt(gn)) * gn + 1e-7
