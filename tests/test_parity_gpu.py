"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Both sides get identical seeded inputs (workloads/): the oracle reads the stored
float32 or bf16 values exactly, promoted to float64. Tolerances (written per
test) follow the arithmetic of the GPU path:
  * fp32 points: potentials within 1e-4 * eps absolute, cost within 1e-5 relative;
  * bf16 points: potentials within 1e-3 * max(|f_ref|_inf, eps), cost 1e-3 relative;
  * gradient and transport application, both sides fed the same fp32 potentials:
    |delta|_inf / |ref|_inf <= 1e-5 (fp32 points) or 1e-3 (bf16 points).
Shapes span several workgroup tiles and column splits and end in ragged tails;
the full-size workloads are checked on sampled rows that the oracle computes one
by one, and through properties that hold at any size.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.golden import fullsize as FS
from tests.golden import newton_cases as NC

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sk():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import streaming_sinkhorn_solver_log_amd as sk
    return sk


DEV = "cuda:0"


def dev_points(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(arr).to(DEV)


def dev(inp):
    return (dev_points(inp.x, inp.w.dtype), dev_points(inp.y, inp.w.dtype),
            torch.from_numpy(inp.a).to(DEV), torch.from_numpy(inp.b).to(DEV))


def tol_pot(w, ref):
    if w.dtype == "bf16":
        return 1e-3 * max(np.abs(ref).max(), w.eps)
    return 1e-4 * w.eps


def tol_rel(w):
    return 1e-3 if w.dtype == "bf16" else 1e-5


def bf16_variant(w, name="bf16"):
    from dataclasses import replace
    return replace(w, dtype="bf16", name=w.name + "_" + name)


SOLVE_CASES = [
    # (config key, n, m, iters or None for the config's own count)
    (1, 1024, 1024, None),        # the tiny configuration at full size
    (1, 1000, 333, 20),
    (2, 1500, 2100, 40),          # symmetric schedule, eps = 0.01
    (6, 2000, 1777, 30),          # alternating, eps = 0.01
    (1, 1, 1, 5),
    (1, 1, 700, 5),
    (1, 700, 1, 5),
    (1, 257, 4099, 10),
    (3, 2000, 1500, 20),          # bf16 points, d = 64, Dirichlet weights
    (3, 129, 2111, 5),
    (4, 600, 700, 5),             # float32 points, d = 512 (GEMM-tiled pass)
    (7, 700, 333, 5),             # bf16 points, d = 512
    (5, 300, 1300, 4),            # bf16 points, d = 1024, rectangular
]


@pytest.mark.parametrize("key,n,m,iters", SOLVE_CASES)
def test_solve_matches_oracle(sk, key, n, m, iters):
    w = W.CASES[key].scaled(n, m, iters)
    say(f"solve cfg={key} n={n} m={m} d={w.d} iters={w.iters} mode={w.mode} eps={w.eps}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    torch.cuda.synchronize()
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    f, g = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    ef, eg = np.abs(f - fr).max(), np.abs(g - gr).max()
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} tol={tol_pot(w, fr):.3e} cost {float(cost):.9g} vs {cr:.9g}")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert abs(float(cost) - cr) <= tol_rel(w) * max(abs(cr), 1e-30)


FORCED_EXACT_CASES = [
    (6, 3000, 2500),   # float32 d = 3, merged records (register-resident kernel)
    (2, 1500, 2000),   # float32 d = 3, symmetric schedule (separate bias records)
    (3, 2000, 3000),   # bf16 d = 64, float32 column biases
    (7, 700, 900),     # bf16 d = 512, GEMM-tiled kernel
    (4, 300, 700),     # float32 d = 512, GEMM-tiled kernel
]


@pytest.mark.parametrize("key,n,m", FORCED_EXACT_CASES)
def test_forced_exact_fallback(sk, key, n, m, monkeypatch):
    """The shifted sweep's exact recomputation of a row block (taken when its shifted
    sum falls below the floor, which the benchmark workloads never reach), forced from
    the host on every shifted pass: the solve still matches the oracle, and its rounding
    differs from the shifted sweep's, so the recomputation really ran."""
    w = W.CASES[key].scaled(n, m, 4)
    say(f"forced exact fallback cfg={key} n={n} m={m} d={w.d} {w.dtype} mode={w.mode}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f0, g0, _ = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    monkeypatch.setenv("FLASHSK_FORCE_EXACT", "1")
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    torch.cuda.synchronize()
    monkeypatch.delenv("FLASHSK_FORCE_EXACT")
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    ef = np.abs(f.cpu().numpy().astype(np.float64) - fr).max()
    eg = np.abs(g.cpu().numpy().astype(np.float64) - gr).max()
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} tol={tol_pot(w, fr):.3e}")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert abs(float(cost) - cr) <= tol_rel(w) * abs(cr)
    assert not (torch.equal(f, f0) and torch.equal(g, g0)), "the forced recomputation did not run"


SMALL_CASES = [
    # (config key, n, m, iters, mode or None, dtype or None, d or None): shapes the one-launch solve serves
    (1, 1024, 1024, None, None, None, None),   # the tiny configuration itself
    (2, 900, 1100, 40, None, None, None),      # symmetric schedule, eps = 0.01
    (1, 1, 1, 5, None, None, None),
    (1, 2048, 2000, 5, None, None, None),      # alternating at its pair limit: points staged per half-pass
    (1, 1448, 1448, 6, "symmetric", None, None),  # averaged at its pair limit: both sides resident
    (1, 4096, 300, 10, "symmetric", None, None),
    (1, 333, 4096, 10, None, None, None),
    (1, 700, 650, 10, None, "bf16", None),
    (4, 500, 600, 10, None, None, 7),          # d = 7: two float4 per staged point
    (4, 600, 400, 10, "symmetric", "bf16", 6),
]


def _small_workload(key, n, m, iters, mode, dtype, d):
    from dataclasses import replace
    w = W.CASES[key]
    if d is not None:
        w = replace(w, d=d, eps=0.5, name=f"{w.name}_d{d}")
    if dtype is not None:
        w = replace(w, dtype=dtype, name=w.name + "_" + dtype)
    if mode is not None:
        w = replace(w, mode=mode)
    return w.scaled(n, m, iters)


@pytest.mark.parametrize("key,n,m,iters,mode,dtype,d", SMALL_CASES)
def test_small_solve_matches_oracle_and_streaming(sk, key, n, m, iters, mode, dtype, d, monkeypatch):
    """The one-launch solve of small problems against the oracle, and against the
    streaming passes (FLASHSK_SMALL_SOLVE=0) on the same inputs."""
    w = _small_workload(key, n, m, iters, mode, dtype, d)
    say(f"small solve cfg={key} n={n} m={m} d={w.d} {w.dtype} iters={w.iters} mode={w.mode} eps={w.eps}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    monkeypatch.setenv("FLASHSK_SMALL_SOLVE", "0")
    fs, gs, cs = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    torch.cuda.synchronize()
    monkeypatch.delenv("FLASHSK_SMALL_SOLVE")
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    f64, g64 = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    ef, eg = np.abs(f64 - fr).max(), np.abs(g64 - gr).max()
    es = max(np.abs(f64 - fs.cpu().numpy()).max(), np.abs(g64 - gs.cpu().numpy()).max())
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} vs streaming {es:.3e} tol={tol_pot(w, fr):.3e}")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert es <= 2 * tol_pot(w, fr)
    assert abs(float(cost) - cr) <= tol_rel(w) * max(abs(cr), 1e-30)


@pytest.mark.parametrize("mode", ["alternating", "symmetric"])
def test_small_solve_batches_and_zero_weights(sk, mode):
    """The one-launch solve continued from its own output in batches is bitwise the
    solve in one batch (its state is (f, g)); zero weights mask their points; it is
    swap-symmetric in the averaged schedule and repeatable."""
    w = W.CASES[1].scaled(800, 900, 12)
    inp = W.make_inputs(w)
    a_np, b_np = inp.a.copy(), inp.b.copy()
    a_np[::7] = 0.0
    b_np[3::5] = 0.0
    a_np /= a_np.sum()
    b_np /= b_np.sum()
    x, y, _, _ = dev(inp)
    a, b = torch.from_numpy(a_np).to(DEV), torch.from_numpy(b_np).to(DEV)
    f, g, c = sk.solve(x, y, a, b, w.eps, 12, mode)
    f1, g1, _ = sk.solve(x, y, a, b, w.eps, 5, mode)
    f2, g2, c2 = sk.solve(x, y, a, b, w.eps, 7, mode, f0=f1, g0=g1)
    assert torch.equal(f, f2) and torch.equal(g, g2) and float(c) == float(c2)
    fa, ga, _ = sk.solve(x, y, a, b, w.eps, 12, mode)
    assert torch.equal(f, fa) and torch.equal(g, ga)
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), a_np, b_np, w.eps, 12, mode)
    assert np.abs(f.cpu().numpy() - fr).max() <= tol_pot(w, fr)
    assert np.abs(g.cpu().numpy() - gr).max() <= tol_pot(w, gr)
    assert abs(float(c) - cr) <= 1e-5 * abs(cr)
    if mode == "symmetric":
        gs, fs, _ = sk.solve(y, x, b, a, w.eps, 12, mode)
        assert torch.equal(f, fs) and torch.equal(g, gs)


GEMM_TILE_CASES = [
    ("128x128", 7, 700, 900),   # bf16 d = 512: more row blocks than the default tile, several splits
    ("128x256", 7, 333, 1500),
    ("128x128", 4, 300, 700),   # float32 d = 512
    ("128x256", 5, 300, 1300),  # bf16 d = 1024, rectangular
]


@pytest.mark.parametrize("tile,key,n,m", GEMM_TILE_CASES)
def test_gemm_tiles_match_oracle(sk, tile, key, n, m, monkeypatch):
    """The smaller workgroup tiles of the GEMM-tiled half-pass (kept for the re-read
    study of the pass) match the oracle like the default one."""
    w = W.CASES[key].scaled(n, m, 5)
    say(f"gemm tile {tile} cfg={key} n={n} m={m} d={w.d} {w.dtype}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    monkeypatch.setenv("FLASHSK_GEMM_TILE", tile)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    torch.cuda.synchronize()
    monkeypatch.delenv("FLASHSK_GEMM_TILE")
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    ef = np.abs(f.cpu().numpy().astype(np.float64) - fr).max()
    eg = np.abs(g.cpu().numpy().astype(np.float64) - gr).max()
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} tol={tol_pot(w, fr):.3e}")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert abs(float(cost) - cr) <= tol_rel(w) * abs(cr)


CUSTOM_DIMS = [("f32", 16), ("f32", 20), ("f32", 32), ("bf16", 100), ("bf16", 8), ("f32", 7),
               ("f32", 64), ("bf16", 200), ("f32", 130)]


@pytest.mark.parametrize("dtype,d", CUSTOM_DIMS)
def test_solve_other_dimensions(sk, dtype, d):
    from dataclasses import replace
    w = replace(W.CASES[4], d=d, dtype=dtype, eps=0.2, name=f"gauss_d{d}_{dtype}").scaled(900, 1100, 10)
    say(f"solve d={d} {dtype}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    ef, eg = np.abs(f.cpu().numpy() - fr).max(), np.abs(g.cpu().numpy() - gr).max()
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} tol={tol_pot(w, fr):.3e}")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert abs(float(cost) - cr) <= tol_rel(w) * abs(cr)


# Every edge of the kernel choice by dimension: record widths of 1, 2, 4 and 8
# MFMA K blocks (float32 points take six bf16 slots per coordinate, bf16 points
# one), the merged layout's limit (float32 d <= 4, bf16 d <= 8, alternating
# schedule), the first GEMM-tiled widths (float32 d = 22, bf16 d = 129) and the
# largest supported d; ragged n and m; both schedules.
BOUNDARY_DIMS = [
    ("f32", 1, "alternating"), ("f32", 2, "symmetric"), ("f32", 4, "alternating"), ("f32", 5, "alternating"),
    ("f32", 6, "symmetric"), ("f32", 10, "alternating"), ("f32", 11, "alternating"), ("f32", 21, "symmetric"),
    ("f32", 22, "alternating"), ("f32", 300, "symmetric"),
    ("bf16", 1, "alternating"), ("bf16", 8, "alternating"), ("bf16", 9, "symmetric"), ("bf16", 16, "alternating"),
    ("bf16", 17, "alternating"), ("bf16", 33, "symmetric"), ("bf16", 65, "alternating"),
    ("bf16", 128, "alternating"), ("bf16", 129, "symmetric"), ("bf16", 4096, "alternating"),
]


@pytest.mark.parametrize("i,case", list(enumerate(BOUNDARY_DIMS)))
def test_dimension_boundaries(sk, i, case):
    """Solve, gradient and both applications at every dimension boundary of the
    kernel choice, on ragged shapes, against the oracle (the applications and the
    gradient with the GPU's potentials fed to both sides)."""
    from dataclasses import replace
    dtype, d, mode = case
    n, m = 97 + (241 * i) % 900, 131 + (367 * i) % 1100
    while n * m * d > 3e8:
        n, m = n // 2 + 1, m // 2 + 1
    w = replace(W.CASES[4], d=d, dtype=dtype, eps=0.2, mode=mode, name=f"edge_d{d}_{dtype}").scaled(n, m, 3)
    say(f"dimension edge {dtype} d={d} {mode} n={n} m={m}")
    inp = W.make_inputs(w, k=5)
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    fn, gn = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    ef, eg = np.abs(fn - fr).max(), np.abs(gn - gr).max()
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr), (ef, eg, tol_pot(w, fr))
    assert abs(float(cost) - cr) <= tol_rel(w) * abs(cr)
    x64, y64 = inp.x64(), inp.y64()
    grad = sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy()
    ref = oracle.grad_x(x64, y64, inp.a, inp.b, gn, w.eps)
    e_g = np.abs(grad - ref).max() / np.abs(ref).max()
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)
    PV = sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy()
    ref1 = oracle.apply(x64, y64, inp.a, inp.b, fn, gn, w.eps, inp.V)
    PtU = sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy()
    ref2 = oracle.apply(x64, y64, inp.a, inp.b, fn, gn, w.eps, inp.U, transpose=True)
    e1 = np.abs(PV - ref1).max() / np.abs(ref1).max()
    e2 = np.abs(PtU - ref2).max() / np.abs(ref2).max()
    say(f"  max|df|={ef:.2e} max|dg|={eg:.2e} grad {e_g:.2e} P.V {e1:.2e} P^T.U {e2:.2e}")
    assert e_g <= tol_rel(w) and e1 <= tol_rel(w) and e2 <= tol_rel(w)


def _random_case(seed):
    """A seeded random shape: n, m in [1, 2600], d over every kernel family,
    either dtype and schedule, eps in [0.05, 1], k in [1, 64]."""
    from dataclasses import replace
    rng = np.random.default_rng([20, seed])
    dtype = ["f32", "bf16"][int(rng.integers(2))]
    d = int(rng.choice([1, 2, 3, 4, 5, 7, 9, 13, 16, 21, 24, 31, 40, 64, 70, 100, 128, 150, 257, 520]))
    n, m = int(rng.integers(1, 2600)), int(rng.integers(1, 2600))
    while n * m * d > 6e7:
        n, m = max(1, n // 2), max(1, m // 2)
    mode = ["alternating", "symmetric"][int(rng.integers(2))]
    eps = float(np.round(rng.uniform(0.05, 1.0), 3))
    k = int(rng.integers(1, 65))
    iters = int(rng.integers(1, 6))
    w = replace(W.CASES[4], d=d, dtype=dtype, eps=eps, mode=mode, name=f"rand{seed}").scaled(n, m, iters)
    return w, k


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(sk, seed):
    """Solve, gradient, P V and P^T U on seeded random shapes against the oracle
    (the gradient and the applications with the GPU's potentials fed to both sides)."""
    w, k = _random_case(seed)
    say(f"random seed={seed} {w.dtype} d={w.d} n={w.n} m={w.m} {w.mode} eps={w.eps} iters={w.iters} k={k}")
    inp = W.make_inputs(w, k=k)
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    fn, gn = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    ef, eg = np.abs(fn - fr).max(), np.abs(gn - gr).max()
    x64, y64 = inp.x64(), inp.y64()
    grad = sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy()
    ref = oracle.grad_x(x64, y64, inp.a, inp.b, gn, w.eps)
    e_g = np.abs(grad - ref).max() / max(np.abs(ref).max(), 1e-30)
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)
    PV = sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy()
    ref1 = oracle.apply(x64, y64, inp.a, inp.b, fn, gn, w.eps, inp.V)
    PtU = sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy()
    ref2 = oracle.apply(x64, y64, inp.a, inp.b, fn, gn, w.eps, inp.U, transpose=True)
    e1 = np.abs(PV - ref1).max() / np.abs(ref1).max()
    e2 = np.abs(PtU - ref2).max() / np.abs(ref2).max()
    say(f"  max|df|={ef:.2e} max|dg|={eg:.2e} (tol {tol_pot(w, fr):.1e}) grad {e_g:.2e} P.V {e1:.2e} P^T.U {e2:.2e}")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert abs(float(cost) - cr) <= tol_rel(w) * max(abs(cr), 1e-30)
    assert e_g <= tol_rel(w) and e1 <= tol_rel(w) and e2 <= tol_rel(w)


def test_solve_bf16_points_small_d(sk):
    w = bf16_variant(W.CASES[1].scaled(900, 1100, 20))
    say("solve bf16 d=3")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, w.mode)
    assert np.abs(f.cpu().numpy() - fr).max() <= tol_pot(w, fr)
    assert np.abs(g.cpu().numpy() - gr).max() <= tol_pot(w, gr)
    assert abs(float(cost) - cr) <= tol_rel(w) * abs(cr)


def test_zero_iterations_and_warm_start_resume(sk):
    w = W.CASES[6].scaled(1300, 1200, 12)
    say("iters=0 and warm-start resume")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f0, g0, c0 = sk.solve(x, y, a, b, w.eps, 0)
    assert torch.count_nonzero(f0) == 0 and torch.count_nonzero(g0) == 0 and float(c0) == 0.0
    f, g, c = sk.solve(x, y, a, b, w.eps, 12)
    f1, g1, _ = sk.solve(x, y, a, b, w.eps, 5)
    f2, g2, c2 = sk.solve(x, y, a, b, w.eps, 7, f0=f1, g0=g1)
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, 12)
    for ff, gg, cc in ((f, g, c), (f2, g2, c2)):
        assert np.abs(ff.cpu().numpy() - fr).max() <= tol_pot(w, fr)
        assert np.abs(gg.cpu().numpy() - gr).max() <= tol_pot(w, gr)
        assert abs(float(cc) - cr) <= 1e-5 * abs(cr)
    # warm start from arbitrary potentials agrees with the oracle started there
    fs, gs = W.random_potentials(1300, 1200, 0.05, seed=5)
    f3, g3, _ = sk.solve(x, y, a, b, w.eps, 3, "symmetric", f0=torch.from_numpy(fs).to(DEV),
                         g0=torch.from_numpy(gs).to(DEV))
    fr3, gr3, _ = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, 3, "symmetric", fs, gs)
    assert np.abs(f3.cpu().numpy() - fr3).max() <= tol_pot(w, fr3)
    assert np.abs(g3.cpu().numpy() - gr3).max() <= tol_pot(w, gr3)


def _zero_weight_workload(case):
    from dataclasses import replace
    if case == "f32_d3":
        return W.CASES[1].scaled(600, 500, 10), None
    if case in ("bf16_d64", "bf16_d64_symmetric"):  # float32 column biases, four K blocks
        return W.CASES[3].scaled(700, 611, 10), ("symmetric" if case.endswith("symmetric") else None)
    # bf16_d16: float32 column biases, one K block
    return replace(W.CASES[4], d=16, dtype="bf16", eps=0.2, name="gauss_d16_bf16").scaled(650, 555, 10), None


@pytest.mark.parametrize("case", ["f32_d3", "bf16_d64", "bf16_d64_symmetric", "bf16_d16"])
def test_zero_weights(sk, case):
    # zero weights give -inf column biases: masked columns that add nothing
    w, mode = _zero_weight_workload(case)
    mode = mode or w.mode
    say(f"zero weights {case} n={w.n} m={w.m} d={w.d} mode={mode}")
    inp = W.make_inputs(w)
    inp.a[::7] = 0.0
    inp.b[3::11] = 0.0
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, mode)
    fr, gr, cr = oracle.solve(inp.x64(), inp.y64(), inp.a, inp.b, w.eps, w.iters, mode)
    ef, eg = np.abs(f.cpu().numpy() - fr).max(), np.abs(g.cpu().numpy() - gr).max()
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} tol={tol_pot(w, fr):.3e}")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert abs(float(cost) - cr) <= tol_rel(w) * abs(cr)


def test_repeatable_and_swap_symmetric(sk):
    w = W.CASES[2].scaled(1200, 1200, 15)
    say("bitwise repeatability, swap symmetry")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    r1 = sk.solve(x, y, a, b, w.eps, w.iters, "symmetric")
    r2 = sk.solve(x, y, a, b, w.eps, w.iters, "symmetric")
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1]) and torch.equal(r1[2], r2[2])
    fs, gs, _ = sk.solve(y, x, b, a, w.eps, w.iters, "symmetric")
    assert torch.equal(fs, r1[1]) and torch.equal(gs, r1[0])


@pytest.mark.parametrize("key,n,m", [(3, 6000, 5000), (7, 700, 900), (6, 3000, 2500)])
def test_bitwise_repeatable_all_kernels(sk, key, n, m):
    """Every kernel family (register-resident, LDS-staged, GEMM-tiled half-pass; gradient;
    transport application) gives bitwise identical results on repeated calls."""
    w = W.CASES[key].scaled(n, m, 4)
    say(f"repeatability cfg={key} n={n} m={m} d={w.d} {w.dtype}")
    inp = W.make_inputs(w, k=16)
    x, y, a, b = dev(inp)
    V = torch.from_numpy(inp.V).to(DEV)
    ref = None
    for _ in range(4):
        f, g, c = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
        gr = sk.eot_grad_x(x, y, a, b, g, w.eps)
        pv = sk.transport_apply(x, y, a, b, f, g, w.eps, V)
        cur = (f, g, c, gr, pv)
        if ref is None:
            ref = cur
        else:
            for r, t in zip(ref, cur):
                assert torch.equal(r, t)


def test_side_streams_and_caller_workspace(sk):
    """Work is ordered on the caller's current stream only: two problems of
    different kernel families issued on two side streams without any host
    synchronization in between give bitwise the default-stream results, also
    when every call takes a caller workspace pre-filled with 0xFF (the library
    initializes every counter and partial it relies on)."""
    cases = [(3, 6000, 5000), (6, 3000, 2500)]
    probs, refs = [], []
    for key, n, m in cases:
        w = W.CASES[key].scaled(n, m, 6)
        say(f"side streams cfg={key} n={n} m={m} d={w.d} {w.dtype}")
        inp = W.make_inputs(w, k=16)
        x, y, a, b = dev(inp)
        V = torch.from_numpy(inp.V).to(DEV)
        f, g, c = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
        refs.append((f, g, c, sk.eot_grad_x(x, y, a, b, g, w.eps),
                     sk.transport_apply(x, y, a, b, f, g, w.eps, V)))
        probs.append((w, x, y, a, b, V))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    outs = []
    for (w, x, y, a, b, V), s in zip(probs, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            ws = torch.full((1 << 26,), 255, dtype=torch.uint8, device=DEV)
            f, g, c = sk.solve(x, y, a, b, w.eps, w.iters, w.mode, workspace=ws)
            ws.fill_(255)
            gr = sk.eot_grad_x(x, y, a, b, g, w.eps, workspace=ws)
            ws.fill_(255)
            pv = sk.transport_apply(x, y, a, b, f, g, w.eps, V, workspace=ws)
            outs.append((f, g, c, gr, pv))
    torch.cuda.synchronize()
    for ref, out in zip(refs, outs):
        for r, t in zip(ref, out):
            assert torch.equal(r, t)


def test_check_finite_screens_inputs(sk):
    """SK_CHECK_FINITE: clean inputs give bitwise the unchecked result; a NaN
    or an infinity in the points, a negative or NaN weight, an all-zero
    marginal or a non-finite warm start is refused with SK_ERR_INVALID_ARG."""
    nan, inf = float("nan"), float("inf")
    for key in (1, 3, 4):  # float32 d = 3, bf16 d = 64, float32 d = 512 (GEMM-tiled)
        w = W.CASES[key].scaled(700, 900, 5)
        say(f"check_finite cfg={key} {w.dtype} d={w.d}")
        inp = W.make_inputs(w)
        x, y, a, b = dev(inp)
        ref = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
        out = sk.solve(x, y, a, b, w.eps, w.iters, w.mode, check_finite=True)
        for r, t in zip(ref, out):
            assert torch.equal(r, t)
        f0, g0 = ref[0].clone(), ref[1].clone()

        def put(t, idx, v):
            t = t.clone()
            t[idx] = v
            return t
        bad = {
            "nan in x": dict(x=put(x, (17, 1 % w.d), nan)),
            "inf in y": dict(y=put(y, (899, 0), -inf)),
            "negative a": dict(a=put(a, 3, -1e-6)),
            "nan in b": dict(b=put(b, 0, nan)),
            "all-zero a": dict(a=torch.zeros_like(a)),
            "inf in f0": dict(f0=put(f0, 5, inf), g0=g0),
        }
        for name, over in bad.items():
            args = dict(x=x, y=y, a=a, b=b)
            args.update(over)
            with pytest.raises(sk.SinkhornError) as err:
                sk.solve(args.pop("x"), args.pop("y"), args.pop("a"), args.pop("b"), w.eps, w.iters, w.mode,
                         check_finite=True, **args)
            assert err.value.code == sk.SK_ERR_INVALID_ARG, name
        # the same warm start, finite, is accepted
        sk.solve(x, y, a, b, w.eps, 1, w.mode, f0=f0, g0=g0, check_finite=True)


def test_translation_invariance(sk):
    w = W.CASES[1].scaled(800, 900, 10)
    say("translation invariance")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    t = torch.tensor([3.0, -7.0, 11.0], device=DEV)
    f1, g1, c1 = sk.solve(x, y, a, b, w.eps, w.iters)
    f2, g2, c2 = sk.solve(x + t, y + t, a, b, w.eps, w.iters)
    assert (f1 - f2).abs().max().item() <= 1e-4 * w.eps
    assert abs(float(c1) - float(c2)) <= 1e-5 * abs(float(c1))


@pytest.mark.parametrize("mode", ["alternating", "symmetric"])
def test_bf16_clouds_far_from_the_origin(sk, mode, monkeypatch):
    """bf16 points near 200 in every coordinate: the library translates them by
    an exactly representable shift (bf16 differences stay bf16), so the
    |x|^2 + |y|^2 - 2 x.y expansion keeps its accuracy. Solve, gradient and
    application against the oracle on the same stored values; without the
    shift (center=False) the float32 expansion is visibly worse. The streaming
    passes are forced (the one-launch small solve forms direct differences and
    needs no shift)."""
    monkeypatch.setenv("FLASHSK_SMALL_SOLVE", "0")
    rng = np.random.default_rng([31, 5])
    n, m, d, eps, iters = 700, 900, 8, 1.0, 10
    xs = W.f32_to_bf16_bits((200.0 + 1.5 * rng.standard_normal((n, d))).astype(np.float32))
    ys = W.f32_to_bf16_bits((201.0 + 1.5 * rng.standard_normal((m, d))).astype(np.float32))
    a = np.full(n, np.float32(1.0 / n), dtype=np.float32)
    b = np.full(m, np.float32(1.0 / m), dtype=np.float32)
    x64, y64 = W.bf16_bits_to_f32(xs).astype(np.float64), W.bf16_bits_to_f32(ys).astype(np.float64)
    x, y = dev_points(xs, "bf16"), dev_points(ys, "bf16")
    at, bt = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    say(f"bf16 far from the origin, {mode}")
    f, g, cost = sk.solve(x, y, at, bt, eps, iters, mode)
    fr, gr, cr = oracle.solve(x64, y64, a, b, eps, iters, mode)
    fn, gn = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    ef, eg = np.abs(fn - fr).max(), np.abs(gn - gr).max()
    tol = 1e-3 * max(np.abs(fr).max(), eps)
    f0, g0, _ = sk.solve(x, y, at, bt, eps, iters, mode, center=False)
    e0 = np.abs(f0.cpu().numpy().astype(np.float64) - fr).max()
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} (tol {tol:.1e}); without the shift max|df|={e0:.3e}")
    assert ef <= tol and eg <= tol
    assert abs(float(cost) - cr) <= 1e-3 * abs(cr)
    assert e0 > 10 * ef
    grad = sk.eot_grad_x(x, y, at, bt, g, eps).cpu().numpy()
    ref = oracle.grad_x(x64, y64, a, b, gn, eps)
    e_g = np.abs(grad - ref).max() / np.abs(ref).max()
    V = torch.from_numpy(rng.standard_normal((m, 5)).astype(np.float32)).to(DEV)
    PV = sk.transport_apply(x, y, at, bt, f, g, eps, V).cpu().numpy()
    ref1 = oracle.apply(x64, y64, a, b, fn, gn, eps, V.cpu().numpy())
    e1 = np.abs(PV - ref1).max() / np.abs(ref1).max()
    say(f"  grad rel err {e_g:.3e}, P.V rel err {e1:.3e}")
    assert e_g <= 1e-3 and e1 <= 1e-3


GRAD_CASES = [
    (2, 1500, 2100),   # float32 d = 3, symmetric-schedule potentials
    (1, 1000, 333),    # one column split
    (1, 1, 50),
    (6, 1200, 5000),   # several column splits
    (3, 2000, 1500),   # bf16 d = 64: two value blocks
    (4, 600, 700),     # float32 d = 512: GEMM-tiled, 16 value blocks in 8 chunks
    (7, 500, 333),     # bf16 d = 512
]


@pytest.mark.parametrize("key,n,m", GRAD_CASES)
def test_grad_matches_oracle(sk, key, n, m):
    w = W.CASES[key].scaled(n, m, 10)
    say(f"grad cfg={key} n={n} m={m}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    _, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    grad = sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy()
    ref = oracle.grad_x(inp.x64(), inp.y64(), inp.a, inp.b, g.cpu().numpy().astype(np.float64), w.eps)
    err = np.abs(grad - ref).max() / np.abs(ref).max()
    say(f"  rel err {err:.3e}")
    assert err <= tol_rel(w)


APPLY_CASES = [
    (1, 1000, 333, 16),
    (6, 1200, 1900, 5),
    (1, 1, 40, 3),
    (1, 64, 64, 64),     # two value blocks
    (3, 1000, 1500, 64), # bf16 d = 64
    (3, 500, 3000, 7),
    (5, 300, 1300, 16),  # bf16 d = 1024, GEMM-tiled
    (4, 600, 700, 40),   # float32 d = 512, two value blocks
    (4, 300, 1300, 16),  # float32 d = 512, 8-wave tile: the last column block overhangs the padding
    (4, 300, 700, 130),  # float32 d = 512, wide kernel (two value blocks per wave)
    (7, 250, 900, 600),  # bf16 d = 512, wide kernel, two value chunks
    (3, 400, 500, 100),  # bf16 d = 64, register-resident kernel over two value chunks
    (1, 200, 333, 97),   # float32 d = 3, widths past 64
    (3, 300, 500, 1),    # bf16 d = 64, a single value column (float16 form, shared stages)
    (3, 200, 300, 4096), # bf16 d = 64, the widest application: 64 value chunks
    (6, 200, 300, 4096), # float32 d = 3, the widest application
    (7, 100, 200, 4096), # bf16 d = 512, the widest application on the wide kernel
]


@pytest.mark.parametrize("key,n,m,k", APPLY_CASES)
def test_apply_matches_oracle(sk, key, n, m, k):
    w = W.CASES[key].scaled(n, m, 10)
    say(f"apply cfg={key} n={n} m={m} k={k}")
    inp = W.make_inputs(w, k=k)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    f64, g64 = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)
    PV = sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy()
    PtU = sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy()
    ref = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.V)
    reft = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.U, transpose=True)
    e1 = np.abs(PV - ref).max() / np.abs(ref).max()
    e2 = np.abs(PtU - reft).max() / np.abs(reft).max()
    say(f"  rel err P.V {e1:.3e}  P^T.U {e2:.3e}")
    assert e1 <= tol_rel(w) and e2 <= tol_rel(w)


AUX_DIMS = [("f32", 16), ("f32", 32), ("bf16", 100), ("bf16", 8), ("f32", 7), ("bf16", 200), ("f32", 130)]


@pytest.mark.parametrize("dtype,d", AUX_DIMS)
def test_grad_apply_other_dimensions(sk, dtype, d):
    from dataclasses import replace
    w = replace(W.CASES[4], d=d, dtype=dtype, eps=0.2, name=f"gauss_d{d}_{dtype}").scaled(700, 1300, 5)
    say(f"grad/apply d={d} {dtype}")
    inp = W.make_inputs(w, k=40)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    f64, g64 = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    grad = sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy()
    ref = oracle.grad_x(inp.x64(), inp.y64(), inp.a, inp.b, g64, w.eps)
    eg = np.abs(grad - ref).max() / np.abs(ref).max()
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)
    PV = sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy()
    PtU = sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy()
    ref1 = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.V)
    ref2 = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.U, transpose=True)
    e1 = np.abs(PV - ref1).max() / np.abs(ref1).max()
    e2 = np.abs(PtU - ref2).max() / np.abs(ref2).max()
    say(f"  rel err grad {eg:.3e}  P.V {e1:.3e}  P^T.U {e2:.3e}")
    assert eg <= tol_rel(w) and e1 <= tol_rel(w) and e2 <= tol_rel(w)


@pytest.mark.parametrize("key,scale", [(1, 0.5), (3, 0.3), (4, 2.0)])
def test_apply_arbitrary_potentials(sk, key, scale):
    """Plan entries spread over many orders of magnitude (potentials not from a solve)."""
    w = W.CASES[key].scaled(700, 900, 1)
    say(f"apply cfg={key} arbitrary potentials scale={scale}")
    inp = W.make_inputs(w, k=16)
    x, y, a, b = dev(inp)
    fs, gs = W.random_potentials(w.n, w.m, scale, seed=11)
    f, g = torch.from_numpy(fs).to(DEV), torch.from_numpy(gs).to(DEV)
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)
    PV = sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy()
    PtU = sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy()
    f64, g64 = fs.astype(np.float64), gs.astype(np.float64)
    ref1 = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.V)
    ref2 = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.U, transpose=True)
    # row-wise relative error: each row of P V has its own scale here
    r1 = np.abs(PV - ref1).max(axis=1) / np.maximum(np.abs(ref1).max(axis=1), 1e-300)
    r2 = np.abs(PtU - ref2).max(axis=1) / np.maximum(np.abs(ref2).max(axis=1), 1e-300)
    say(f"  worst row rel err P.V {r1.max():.3e}  P^T.U {r2.max():.3e}")
    tol = 1e-3 if w.dtype == "bf16" else 1e-4
    assert r1.max() <= tol and r2.max() <= tol
    gr = sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy()
    refg = oracle.grad_x(inp.x64(), inp.y64(), inp.a, inp.b, g64, w.eps)
    eg = np.abs(gr - refg).max() / np.abs(refg).max()
    say(f"  grad rel err {eg:.3e}")
    assert eg <= tol_rel(w)


HALF_FORM_CASES = [
    # (config key, eps, k): the transport kernels' float16 form
    (3, 0.1, 21),     # bf16 d = 64, register-resident kernel
    (3, 0.004, 21),   # nearly a permutation plan
    (6, 0.05, 21),    # float32 d = 3 (two float16 parts per entry)
    (7, 0.1, 100),    # bf16 d = 512, k > 64: the wide kernel
    (4, 0.2, 100),    # float32 d = 512, the wide kernel
]


@pytest.mark.parametrize("key,eps,k", HALF_FORM_CASES)
def test_half_precision_form_column_scales(sk, key, eps, k):
    """The transport kernels' half-precision form (float16 parts of the plan
    entries, values as two float16 parts after a power-of-two scale per value
    column). Value columns spanning 10^-30 .. 10^30, a zero column and a
    column mixing magnitudes 2^-40 .. 1 must each keep the configuration's
    bound relative to their own largest output; at eps = 0.004 the plan is
    nearly a permutation, so single entries carry the rounding (2^-11 of an
    entry at most for bf16 points). Shape: several 32-column tiles with
    ragged rows, columns and value width."""
    from dataclasses import replace
    w = replace(W.CASES[key].scaled(700, 900, 1), eps=eps)
    say(f"half-precision form cfg={key} eps={eps} k={k} n={w.n} m={w.m} d={w.d} {w.dtype}")
    inp = W.make_inputs(w, k=k)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, 30, w.mode)
    f64, g64 = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng([key, k, eps > 0.01])
    scales = 10.0 ** np.linspace(-30, 30, k)
    for Vn, nrows in ((inp.V, w.m), (inp.U, w.n)):
        Vn *= scales[None, :].astype(np.float32)
        Vn[:, 3] = 0.0
        Vn[:, 7] = (rng.standard_normal(nrows) * 2.0 ** rng.integers(-40, 1, nrows)).astype(np.float32)
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)
    PV = sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy().astype(np.float64)
    PtU = sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy().astype(np.float64)
    ref1 = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.V)
    ref2 = oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.U, transpose=True)
    for out, ref, what in ((PV, ref1, "P.V"), (PtU, ref2, "P^T.U")):
        assert np.all(out[:, 3] == 0.0)
        den = np.abs(ref).max(axis=0)
        live = den > 0
        col = np.abs(out - ref).max(axis=0)[live] / den[live]
        say(f"  {what}: worst column rel err {col.max():.3e} (column {int(np.argmax(col))})")
        assert col.max() <= tol_rel(w)
    gr = sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy()
    refg = oracle.grad_x(inp.x64(), inp.y64(), inp.a, inp.b, g64, w.eps)
    eg = np.abs(gr - refg).max() / np.abs(refg).max()
    say(f"  grad rel err {eg:.3e}")
    assert eg <= tol_rel(w)


SMALL_AUX_CASES = [
    # (config key, n, m, k, dtype or None, d or None, potentials): shapes the one-launch
    # gradient and applications serve; "solve" = a 10-iteration solve's pair,
    # "random" = potentials spread over orders of magnitude
    (1, 1024, 1024, 16, None, None, "solve"),   # the tiny configuration, k = 16
    (1, 1, 40, 3, None, None, "solve"),
    (1, 333, 4096, 5, None, None, "solve"),     # eight column chunks (P V), ragged rows
    (1, 2048, 2000, 13, None, None, "solve"),   # at the pair limit; k padded to 16
    (1, 700, 650, 8, "bf16", None, "solve"),
    (4, 500, 600, 1, None, 7, "solve"),         # d = 7: two float4 per staged point
    (4, 600, 400, 12, "bf16", 6, "solve"),
    (1, 700, 900, 16, None, None, "random"),
]


@pytest.mark.parametrize("key,n,m,k,dtype,d,pots", SMALL_AUX_CASES)
def test_small_aux_matches_oracle_and_streaming(sk, key, n, m, k, dtype, d, pots, monkeypatch):
    """The one-launch gradient and transport applications of small problems
    against the oracle, and against the streaming kernels (FLASHSK_SMALL_SOLVE=0)
    on the same inputs and potentials."""
    w = _small_workload(key, n, m, 10, None, dtype, d)
    say(f"small aux cfg={key} n={n} m={m} d={w.d} {w.dtype} k={k} potentials={pots}")
    inp = W.make_inputs(w, k=k)
    x, y, a, b = dev(inp)
    if pots == "solve":
        f, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    else:
        fs, gs = W.random_potentials(w.n, w.m, 0.5, seed=11)
        f, g = torch.from_numpy(fs).to(DEV), torch.from_numpy(gs).to(DEV)
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)

    def run():
        return (sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy(),
                sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy(),
                sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy())

    small = run()
    monkeypatch.setenv("FLASHSK_SMALL_SOLVE", "0")
    stream = run()
    torch.cuda.synchronize()
    monkeypatch.delenv("FLASHSK_SMALL_SOLVE")
    f64, g64 = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    refs = (oracle.grad_x(inp.x64(), inp.y64(), inp.a, inp.b, g64, w.eps),
            oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.V),
            oracle.apply(inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps, inp.U, transpose=True))
    for name, sm, st, ref in zip(("grad", "P.V", "P^T.U"), small, stream, refs):
        if pots == "random" and name != "grad":
            # row-wise relative error: each row has its own scale here
            den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
            es = (np.abs(sm - ref).max(axis=1) / den).max()
            et = (np.abs(sm - st).max(axis=1) / den).max()
            tol = 1e-3 if w.dtype == "bf16" else 1e-4
        else:
            den = np.abs(ref).max()
            es, et = np.abs(sm - ref).max() / den, np.abs(sm - st).max() / den
            tol = tol_rel(w)
        say(f"  {name}: rel err {es:.3e} vs streaming {et:.3e} (tol {tol:.0e})")
        assert es <= tol and et <= 2 * tol


def _check_last_iteration(sk, w, inp, x, y, a, b, T, mode, rows, cols, tag):
    """(f_T, g_T) = solve(T) and (f', g') = solve(T + 1) from the same cold start.
    Runs are bitwise deterministic, so the first T iterations of the second solve
    are the first solve; its last iteration runs the shifted sweep (every pass after
    a side's first), in the launch configuration of a T + 1 iteration solve. On
    sampled rows and columns, f' and g' are compared with the oracle's maps at the
    GPU's own pair:
      alternating: f' = F(g_T) and g' = G(f');
      symmetric:   f' = (f_T + F(g_T)) / 2 and g' = (g_T + G(f_T)) / 2.
    The cost of the returned pair is compared with <a, f'> + <b, g'> in float64."""
    fT, gT, _ = sk.solve(x, y, a, b, w.eps, T, mode)
    f1, g1, cost = sk.solve(x, y, a, b, w.eps, T + 1, mode)
    assert torch.isfinite(f1).all() and torch.isfinite(g1).all()
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    fT, gT, f1n, g1n = t(fT), t(gT), t(f1), t(g1)
    x64, y64 = inp.x64(), inp.y64()
    Fr = oracle.F(x64[rows], y64, inp.b, gT, w.eps)
    if mode == "alternating":
        fr = Fr
        gr = oracle.G(x64, y64[cols], inp.a, f1n, w.eps)
    else:
        fr = 0.5 * (fT[rows] + Fr)
        gr = 0.5 * (gT[cols] + oracle.G(x64, y64[cols], inp.a, fT, w.eps))
    ef = np.abs(f1n[rows] - fr).max()
    eg = np.abs(g1n[cols] - gr).max()
    tf, tg = tol_pot(w, fr), tol_pot(w, gr)
    s64 = float(np.dot(inp.a.astype(np.float64), f1n) + np.dot(inp.b.astype(np.float64), g1n))
    scale = float(np.abs(inp.a * f1n).sum() + np.abs(inp.b * g1n).sum())
    ec = abs(float(cost) - s64)
    say(f"  {tag}: iteration {T + 1} ({mode}) sampled max|df|={ef:.3e} (tol {tf:.1e}) "
        f"max|dg|={eg:.3e} (tol {tg:.1e}); cost {float(cost):.10g} vs <a,f>+<b,g> {s64:.10g}")
    assert ef <= tf and eg <= tg
    assert ec <= 1e-9 * max(scale, 1e-300)
    return f1, g1, f1n, g1n


SPLIT_SHAPES = [
    (6, 200_000, 700),    # far more row blocks than resident workgroups; 6 stages -> one column chunk
    (6, 700, 200_000),    # few row blocks, many stages: every row block merged from many partials
    (3, 130_000, 900),    # bf16 d = 64, wide row range
    (3, 900, 130_000),    # bf16 d = 64, several column chunks per row block
    (1, 300, 300),        # a single workgroup per side
    (1, 33, 4000),
]


@pytest.mark.parametrize("key,n,m", SPLIT_SHAPES)
def test_work_split_regimes(sk, key, n, m):
    """Shapes at the edges of the balanced work split: the last iteration of a
    4-iteration solve (shifted sweep) on sampled rows and columns."""
    w = W.CASES[key].scaled(n, m, 3)
    say(f"work split cfg={key} n={n} m={m} d={w.d} {w.dtype}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(n, min(n, 64), replace=False))
    cols = np.sort(rng.choice(m, min(m, 64), replace=False))
    _check_last_iteration(sk, w, inp, x, y, a, b, w.iters, "alternating", rows, cols, "work split")


@pytest.mark.parametrize("key", [2, 3, 4, 5, 6, 7])
def test_full_size_sampled_rows(sk, key):
    """Every configuration at full size, in the benchmark's launch configuration:
    the last iteration of the configured solve (the shifted sweep: at n = m = 50k
    and d = 64 over two column chunks, at n = m = 10k both half-passes of the
    averaged schedule in one launch, at d >= 512 the GEMM-tiled passes), then the
    gradient and both applications at the returned pair, checked on sampled rows
    and columns that the oracle computes one by one."""
    w = W.CASES[key]
    say(f"full size cfg={key} n={w.n} m={w.m} d={w.d} {w.dtype} iters={w.iters} mode={w.mode}")
    inp = W.make_inputs(w, k=16)
    x, y, a, b = dev(inp)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(w.n, 96, replace=False))
    cols = np.sort(rng.choice(w.m, 96, replace=False))
    f1, g1, f1n, g1n = _check_last_iteration(sk, w, inp, x, y, a, b, w.iters - 1, w.mode, rows, cols,
                                             "full size")
    x64, y64 = inp.x64(), inp.y64()
    if w.mode == "alternating":
        # the last half-pass was the g-pass: the plan's column sums are b
        colsum = sk.transport_apply(x, y, a, b, f1, g1, w.eps, torch.ones(w.n, device=DEV), transpose=True)
        rel = ((colsum - b).abs() / b).max().item()
        say(f"  column-sum rel err {rel:.3e}")
        assert rel <= max(1e-4, tol_rel(w))
    # gradient (final g) and the applications (GPU potentials fed to both sides)
    a_s = inp.a[rows]
    grad = sk.eot_grad_x(x, y, a, b, g1, w.eps).cpu().numpy()[rows]
    ref = oracle.grad_x(x64[rows], y64, a_s, inp.b, g1n, w.eps)
    e_g = np.abs(grad - ref).max() / np.abs(ref).max()
    V, U = torch.from_numpy(inp.V).to(DEV), torch.from_numpy(inp.U).to(DEV)
    PV = sk.transport_apply(x, y, a, b, f1, g1, w.eps, V).cpu().numpy()[rows]
    ref1 = oracle.apply(x64[rows], y64, a_s, inp.b, f1n[rows], g1n, w.eps, inp.V)
    PtU = sk.transport_apply(x, y, a, b, f1, g1, w.eps, U, transpose=True).cpu().numpy()[cols]
    ref2 = oracle.apply(x64, y64[cols], inp.a, inp.b[cols], f1n, g1n[cols], w.eps, inp.U, transpose=True)
    e1 = np.abs(PV - ref1).max() / np.abs(ref1).max()
    e2 = np.abs(PtU - ref2).max() / np.abs(ref2).max()
    say(f"  sampled rel err grad {e_g:.3e}  P.V {e1:.3e}  P^T.U {e2:.3e} (tol {tol_rel(w):.0e})")
    assert e_g <= tol_rel(w) and e1 <= tol_rel(w) and e2 <= tol_rel(w)


@pytest.mark.parametrize("key", FS.KEYS)
def test_full_size_against_stored_oracle(sk, key):
    """End to end at full size: the configured solve against the float64 oracle's
    own solve of the same inputs (stored by tests/golden/make_oracle_fullsize.py,
    keyed by digests of the inputs and of the oracle source): every entry of f and
    g, and the cost. Then the gradient and applications from the GPU's own
    potentials against the oracle's from its own; their bounds add, to the
    tolerance of a single evaluation, what the potential differences measured
    here can move a plan entry: |dP_ij| <= P_ij (exp((|df_i| + |dg_j|)/eps) - 1),
    and a softmax weight of the gradient at most by exp(2 |dg|_inf / eps) - 1."""
    w = W.CASES[key]
    ref = FS.load(w)
    if ref is None:
        pytest.skip(f"no stored reference for {w.name} (tests/golden/make_oracle_fullsize.py)")
    inp = W.make_inputs(w)
    meta = ref["meta"]
    assert meta["input_sha256"] == FS.input_digest(inp), "inputs changed: the stored reference is stale"
    assert meta["oracle_sha256"] == FS.oracle_digest(), "oracle changed: the stored reference is stale"
    say(f"stored oracle cfg={key} n={w.n} m={w.m} d={w.d} {w.dtype} iters={w.iters} mode={w.mode}")
    x, y, a, b = dev(inp)
    f, g, cost = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    fn, gn = t(f), t(g)
    fr, gr, cr = ref["f"], ref["g"], float(ref["cost"])
    dfv, dgv = np.abs(fn - fr), np.abs(gn - gr)
    ef, eg = dfv.max(), dgv.max()
    # gauge-free view (the (c, -c) direction is neutral under both maps)
    c = float(np.dot(inp.a, fn - fr))
    eq = max(np.abs(fn - fr - c).max(), np.abs(gn - gr + c).max())
    ec = abs(float(cost) - cr) / abs(cr)
    say(f"  max|df|={ef:.3e} max|dg|={eg:.3e} (tol {tol_pot(w, fr):.1e}; gauge-free {eq:.3e}) "
        f"cost {float(cost):.10g} vs {cr:.10g} rel {ec:.2e} (tol {tol_rel(w):.0e})")
    assert ef <= tol_pot(w, fr) and eg <= tol_pot(w, gr)
    assert ec <= tol_rel(w)
    x64, y64 = inp.x64(), inp.y64()
    if "grad" in ref:
        rows = ref["grad_rows"]
        grad = sk.eot_grad_x(x, y, a, b, g, w.eps).cpu().numpy()[rows].astype(np.float64)
        gref = ref["grad"]
        dg = gn - gr  # the softmax over j ignores a constant shift of g
        spread = np.expm1(2.0 * 0.5 * (dg.max() - dg.min()) / w.eps)
        reach = np.abs(y64).max(axis=0)[None, :] + np.abs(x64[rows])
        bound = tol_rel(w) * np.abs(gref).max() + 2.0 * inp.a[rows, None] * spread * reach
        worst = (np.abs(grad - gref) / bound).max()
        say(f"  gradient rows {len(rows)}: max|d|={np.abs(grad - gref).max():.3e}, worst share of bound {worst:.3f}")
        assert worst <= 1.0
    if "pv" in ref:
        inpk = W.make_inputs(w, k=w.apply_k)
        V, U = torch.from_numpy(inpk.V).to(DEV), torch.from_numpy(inpk.U).to(DEV)
        rows, cols = ref["pv_rows"], ref["ptu_cols"]
        PV = sk.transport_apply(x, y, a, b, f, g, w.eps, V).cpu().numpy()[rows]
        PtU = sk.transport_apply(x, y, a, b, f, g, w.eps, U, transpose=True).cpu().numpy()[cols]
        b1 = tol_rel(w) * np.abs(ref["pv"]).max() + np.expm1((dfv[rows, None] + eg) / w.eps) * ref["pv_abs"]
        b2 = tol_rel(w) * np.abs(ref["ptu"]).max() + np.expm1((dgv[cols, None] + ef) / w.eps) * ref["ptu_abs"]
        w1 = (np.abs(PV - ref["pv"]) / b1).max()
        w2 = (np.abs(PtU - ref["ptu"]) / b2).max()
        say(f"  P.V rows {len(rows)} worst share of bound {w1:.3f}; P^T.U cols {len(cols)} {w2:.3f}")
        assert w1 <= 1.0 and w2 <= 1.0


DIV_CASES = [
    # (config key, n, m, iters)
    (2, 700, 900, 20),   # float32 d = 3, symmetric cross term
    (6, 500, 1300, 15),  # float32 d = 3, alternating, merged records
    (3, 600, 800, 10),   # bf16 d = 64
    (4, 300, 400, 5),    # float32 d = 512 (GEMM-tiled)
    (5, 200, 700, 4),    # bf16 d = 1024, rectangular
]


@pytest.mark.parametrize("key,n,m,iters", DIV_CASES)
def test_divergence_matches_oracle(sk, key, n, m, iters):
    """Debiased divergence: the device composition is checked exactly against the
    same solves run through the solve entry point (bitwise repeatable), the
    gradients in x and y against the oracle fed those potentials, and S and the
    weight gradients end to end against the oracle's own solves."""
    w = W.CASES[key].scaled(n, m, iters)
    say(f"divergence cfg={key} n={n} m={m} iters={iters} {w.dtype} d={w.d}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    S, ga, gb, gx, gy = sk.sinkhorn_divergence(x, y, a, b, w.eps, w.iters, w.mode)
    f_ab, g_ab, c_ab = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    f_aa, g_aa, c_aa = sk.solve(x, x, a, a, w.eps, w.iters, "symmetric")
    f_bb, g_bb, c_bb = sk.solve(y, y, b, b, w.eps, w.iters, "symmetric")
    c = [float(v) for v in (c_ab, c_aa, c_bb)]
    assert float(S) == c[0] - 0.5 * c[1] - 0.5 * c[2]
    assert torch.equal(ga, f_ab - f_aa) and torch.equal(gb, g_ab - g_bb)
    x64, y64 = inp.x64(), inp.y64()
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    cross_x = oracle.grad_x(x64, y64, inp.a, inp.b, t(g_ab), w.eps)
    self_x = oracle.grad_x(x64, x64, inp.a, inp.a, t(g_aa), w.eps)
    cross_y = oracle.grad_x(y64, x64, inp.b, inp.a, t(f_ab), w.eps)
    self_y = oracle.grad_x(y64, y64, inp.b, inp.b, t(g_bb), w.eps)
    ex = np.abs(t(gx) - (cross_x - self_x)).max() / max(np.abs(cross_x).max(), np.abs(self_x).max())
    ey = np.abs(t(gy) - (cross_y - self_y)).max() / max(np.abs(cross_y).max(), np.abs(self_y).max())
    S_ref, ga_ref, gb_ref, _, _ = oracle.divergence(x64, y64, inp.a, inp.b, w.eps, w.iters, w.mode)
    # S is a difference of costs: its error bound is the cost tolerance times their magnitudes
    tol_s = tol_rel(w) * (abs(c[0]) + 0.5 * abs(c[1]) + 0.5 * abs(c[2]))
    es = abs(float(S) - S_ref)
    ea = np.abs(t(ga) - ga_ref).max()
    eb = np.abs(t(gb) - gb_ref).max()
    ta, tb = 2 * tol_pot(w, ga_ref), 2 * tol_pot(w, gb_ref)
    say(f"  S={float(S):.6e} ref={S_ref:.6e} |dS|={es:.2e} (tol {tol_s:.1e}); grad_a {ea:.2e} (tol {ta:.1e}) "
        f"grad_b {eb:.2e} (tol {tb:.1e}); grad_x {ex:.2e} grad_y {ey:.2e} (tol {tol_rel(w):.0e})")
    assert es <= tol_s and ea <= ta and eb <= tb
    assert ex <= tol_rel(w) and ey <= tol_rel(w)
    # without gradients only S is written
    S2, *rest = sk.sinkhorn_divergence(x, y, a, b, w.eps, w.iters, w.mode, grads=False)
    assert float(S2) == float(S) and all(r is None for r in rest)


HADAMARD_CASES = [
    # (config key, n, m, r, k)
    (1, 300, 500, 3, 5),      # one group of ranks
    (6, 700, 400, 20, 8),     # three groups (8 ranks of width 8 per application), the last partial
    (3, 500, 900, 4, 16),     # bf16 d = 64
    (4, 200, 300, 2, 33),     # float32 d = 512 (GEMM-tiled), two value blocks
    (1, 1, 70, 1, 1),         # a single row
]


@pytest.mark.parametrize("key,n,m,r,k", HADAMARD_CASES)
def test_hadamard_apply_matches_oracle(sk, key, n, m, r, k):
    """(P o A B^T) V and its transpose against the oracle's entrywise definition,
    both sides fed the same float32 potentials; the bound is relative to
    |P| |W| |V| (signed weights may cancel)."""
    w = W.CASES[key].scaled(n, m, 8)
    say(f"hadamard apply cfg={key} n={n} m={m} r={r} k={k}")
    inp = W.make_inputs(w, k=k)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    rng = np.random.default_rng([key, n, r, k])
    A = rng.standard_normal((n, r)).astype(np.float32)
    B = rng.standard_normal((m, r)).astype(np.float32)
    f64, g64 = f.cpu().numpy().astype(np.float64), g.cpu().numpy().astype(np.float64)
    args = (inp.x64(), inp.y64(), inp.a, inp.b, f64, g64, w.eps)
    At, Bt = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    for transpose, vals in ((False, inp.V), (True, inp.U)):
        out = sk.transport_apply_hadamard(x, y, a, b, f, g, w.eps, At, Bt, torch.from_numpy(vals).to(DEV),
                                          transpose=transpose).cpu().numpy()
        ref = oracle.apply_hadamard(*args, A, B, vals, transpose=transpose)
        scale = np.abs(oracle.apply_hadamard(*args, np.abs(A), np.abs(B), np.abs(vals), transpose=transpose)).max()
        err = np.abs(out - ref).max() / scale
        say(f"  transpose={int(transpose)} rel err {err:.3e} (tol {tol_rel(w):.0e})")
        assert err <= tol_rel(w)


@pytest.mark.parametrize("mode", ["symmetric", "alternating"])
def test_solve_tol_error_matches_oracle(sk, mode):
    """The marginal error the tolerance solve measures equals the oracle's
    ||P1 - a||_1 + ||P^T 1 - b||_1 at the checked pair (far from convergence)."""
    w = W.CASES[6].scaled(900, 700, 3)
    say(f"solve_tol error parity mode={mode}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, 3, mode)
    if mode == "symmetric":
        # the check runs on the starting pair itself
        _, _, _, done, err = sk.solve_tol(x, y, a, b, w.eps, 0.0, 1, mode, check_every=1, f0=f, g0=g)
        fc, gc = f, g
    else:
        # one iteration produces the checked pair (its columns exact), the next measures it
        _, _, _, done, err = sk.solve_tol(x, y, a, b, w.eps, 0.0, 2, mode, check_every=2, f0=f, g0=g)
        fc, gc, _ = sk.solve(x, y, a, b, w.eps, 1, mode, f0=f, g0=g)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    r, c = oracle.marginals(inp.x64(), inp.y64(), inp.a, inp.b, t(fc), t(gc), w.eps)
    ref = np.abs(r - inp.a).sum() + np.abs(c - inp.b).sum()
    say(f"  iters {done} err {err:.6e} ref {ref:.6e}")
    assert done == (1 if mode == "symmetric" else 2)
    assert err == pytest.approx(ref, rel=1e-3, abs=1e-6)


@pytest.mark.parametrize("key,n,m", [(1, 600, 500), (3, 400, 700), (6, 800, 700)])
def test_solve_tol_reaches_tolerance(sk, key, n, m):
    w = W.CASES[key].scaled(n, m)
    say(f"solve_tol convergence cfg={key} n={n} m={m} {w.dtype}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    tol = 1e-4
    f, g, cost, done, err = sk.solve_tol(x, y, a, b, w.eps, tol, 5000, check_every=10)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    r, c = oracle.marginals(inp.x64(), inp.y64(), inp.a, inp.b, t(f), t(g), w.eps)
    ref = np.abs(r - inp.a).sum() + np.abs(c - inp.b).sum()
    say(f"  iters {done} err {err:.3e}; oracle marginal error of the returned pair {ref:.3e}")
    assert done < 5000 and done % 10 == 0 and err <= tol and ref <= tol
    # with tol = 0 it runs to max_iters
    _, _, _, done0, err0 = sk.solve_tol(x, y, a, b, w.eps, 0.0, 35, check_every=10)
    assert done0 == 35 and np.isfinite(err0)


HVP_CASES = [
    # (config key, n, m, eps override or None)
    (1, 300, 400, 0.1),      # float32 d = 3
    (6, 500, 450, 0.05),     # float32 d = 3, mixture
    (3, 300, 350, None),     # bf16 d = 64
    (2, 200, 260, 0.02),     # float32 d = 3, smaller eps
    (4, 120, 150, None),     # float32 d = 512 (GEMM-tiled records)
    (7, 110, 130, None),     # bf16 d = 512
    (5, 60, 200, None),      # bf16 d = 1024, rectangular
]


@pytest.mark.parametrize("key,n,m,eps", HVP_CASES)
def test_hvp_matches_dense_oracle(sk, key, n, m, eps):
    """Streaming Hessian-vector product (Schur CG over matrix-free applications)
    against the oracle's dense Moore-Penrose solve at the same (converged) pair."""
    from dataclasses import replace
    w = W.CASES[key].scaled(n, m, 300)
    if eps is not None:
        w = replace(w, eps=eps)
    say(f"hvp cfg={key} n={n} m={m} d={w.d} {w.dtype} eps={w.eps}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, "alternating")
    V = np.random.default_rng([key, n, 3]).standard_normal((n, w.d)).astype(np.float32)
    HV, iters, resid = sk.ot_hvp_x(x, y, a, b, f, g, w.eps, torch.from_numpy(V).to(DEV), cg_tol=1e-6)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    ref = oracle.hvp_x(inp.x64(), inp.y64(), inp.a, inp.b, t(f), t(g), w.eps, V)
    err = np.abs(t(HV) - ref).max() / np.abs(ref).max()
    say(f"  CG iterations {iters}, residual {resid:.2e}; rel err {err:.3e}")
    # CG to 1e-6 over float32 applications (1e-5 each) through the Schur system
    assert resid <= 1e-6 and err <= (1e-4 if w.dtype == "f32" else 1e-3)


HVP_EPS = [0.5, 0.2, 0.1, 0.05, 0.02, 0.01, 0.005]


@pytest.mark.parametrize("eps", HVP_EPS)
def test_hvp_eps_sweep_against_dense_oracle(sk, eps):
    """HVP accuracy against eps (the replication review reports the streaming
    HVP within 1% of a dense reference down to eps = 0.01): the mixture geometry
    of the 10k configuration at n = 256, m = 293, the pair solved to a marginal
    error of 1e-5 (or 20000 iterations), CG to 1e-6 (at most 500 iterations),
    against the oracle's dense Moore-Penrose solve at the same pair. As eps
    falls the plan approaches a permutation and the Schur complement a
    singular matrix: the CG needs more iterations and float32 applications
    bound the residual it reaches."""
    from dataclasses import replace
    w = replace(W.CASES[2], eps=eps, mode="alternating").scaled(256, 293)
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, _, done, merr = sk.solve_tol(x, y, a, b, eps, 1e-5, 20000, "alternating", 10)
    V = np.random.default_rng([2, 256, 5]).standard_normal((256, w.d)).astype(np.float32)
    HV, iters, resid = sk.ot_hvp_x(x, y, a, b, f, g, eps, torch.from_numpy(V).to(DEV), cg_tol=1e-6,
                                   cg_max_iters=500)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    ref = oracle.hvp_x(inp.x64(), inp.y64(), inp.a, inp.b, t(f), t(g), eps, V)
    err = np.abs(t(HV) - ref).max() / np.abs(ref).max()
    say(f"hvp eps sweep eps={eps:g}: pair after {done} iterations (marginal error {merr:.1e}); "
        f"CG {iters} iterations, residual {resid:.1e}; max rel err {err:.3e}")
    # the pages' bar is 1e-2; measured 2e-6 (eps = 0.5) to 1.1e-4 (eps = 0.005)
    assert err <= 1e-3


@pytest.mark.parametrize("key", [6, 3])
def test_hvp_full_size_symmetric(sk, key):
    """The HVP at full size (n = m = 50k: the float32 d = 3 mixture at
    eps = 0.01, bf16 d = 64), where the dense oracle cannot run: the Hessian
    of OT_eps in x is symmetric, so <U, H V> = <V, H U> for any tangents U, V
    (review, Summary and Strengths: Theorem 5's Schur solve), and the CG
    reaches its tolerance (the float32 applications in the float16 form do;
    in three bf16 parts they stalled near 1e-2 on the d = 3 mixture)."""
    w = W.CASES[key]
    say(f"hvp full size cfg={key} n={w.n} m={w.m} d={w.d} {w.dtype} eps={w.eps}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, w.mode)
    rng = np.random.default_rng([key, 7])
    U = rng.standard_normal((w.n, w.d)).astype(np.float32)
    V = rng.standard_normal((w.n, w.d)).astype(np.float32)
    HV, itv, rv = sk.ot_hvp_x(x, y, a, b, f, g, w.eps, torch.from_numpy(V).to(DEV), cg_tol=1e-6)
    HU, itu, ru = sk.ot_hvp_x(x, y, a, b, f, g, w.eps, torch.from_numpy(U).to(DEV), cg_tol=1e-6)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    lhs = float((U.astype(np.float64) * t(HV)).sum())
    rhs = float((V.astype(np.float64) * t(HU)).sum())
    rel = abs(lhs - rhs) / max(abs(lhs), abs(rhs))
    say(f"  CG {itv} / {itu} iterations, residuals {rv:.2e} / {ru:.2e}; <U,HV> {lhs:.6e} <V,HU> {rhs:.6e} "
        f"relative asymmetry {rel:.2e}")
    assert rv <= 1e-6 and ru <= 1e-6
    # float32 applications (2^-22 per entry) and bf16 points' two bf16 parts
    # (2^-16), each through a CG solved to 1e-6; measured 2.6e-6 and 2.3e-6
    assert rel <= (1e-4 if w.dtype == "f32" else 1e-3)


@pytest.mark.parametrize("key,n,m,mode", [(6, 1500, 1300, "alternating"), (2, 900, 1100, "symmetric"),
                                           (3, 1200, 1000, "alternating"), (4, 300, 500, "symmetric")])
def test_solve_tol_continues_the_solve(sk, key, n, m, mode):
    """The tolerance solve runs its iterations in one workspace lifetime (one
    prep, shifted sweeps across the checks): with tol = 0 it returns bitwise the
    pair and cost of a plain solve of the same length, cold and warm, whatever
    the check interval."""
    w = W.CASES[key].scaled(n, m, 23)
    say(f"solve_tol continuity cfg={key} n={n} m={m} d={w.d} {w.dtype} {mode}")
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    ref = sk.solve(x, y, a, b, w.eps, 23, mode)
    for every in (1, 4, 10, 23, 40):
        f, g, c, done, err = sk.solve_tol(x, y, a, b, w.eps, 0.0, 23, mode, check_every=every)
        assert done == 23 and torch.equal(f, ref[0]) and torch.equal(g, ref[1]) and torch.equal(c, ref[2]), every
    f0, g0, _ = sk.solve(x, y, a, b, w.eps, 5, mode)
    ref_w = sk.solve(x, y, a, b, w.eps, 12, mode, f0=f0, g0=g0)
    f, g, c, done, err = sk.solve_tol(x, y, a, b, w.eps, 0.0, 12, mode, check_every=5, f0=f0, g0=g0)
    assert done == 12 and torch.equal(f, ref_w[0]) and torch.equal(g, ref_w[1]) and torch.equal(c, ref_w[2])


def test_check_finite_in_composed_operations(sk):
    """SK_CHECK_FINITE reaches the tolerance solve and the divergence: clean
    inputs give bitwise the unchecked results, a NaN point or a negative
    weight is refused with SK_ERR_INVALID_ARG."""
    w = W.CASES[1].scaled(600, 700, 6)
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    r1 = sk.solve_tol(x, y, a, b, w.eps, 1e-3, 40)
    r2 = sk.solve_tol(x, y, a, b, w.eps, 1e-3, 40, check_finite=True)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1]) and r1[3] == r2[3]
    d1 = sk.sinkhorn_divergence(x, y, a, b, w.eps, w.iters)
    d2 = sk.sinkhorn_divergence(x, y, a, b, w.eps, w.iters, check_finite=True)
    assert all(torch.equal(p, q) for p, q in zip(d1, d2))
    xb = x.clone()
    xb[3, 1] = float("nan")
    ab = a.clone()
    ab[7] = -1e-6
    for args in ((xb, y, a, b), (x, y, ab, b)):
        with pytest.raises(sk.SinkhornError) as e1:
            sk.solve_tol(*args, w.eps, 1e-3, 40, check_finite=True)
        with pytest.raises(sk.SinkhornError) as e2:
            sk.sinkhorn_divergence(*args, w.eps, w.iters, check_finite=True)
        assert e1.value.code == sk.SK_ERR_INVALID_ARG and e2.value.code == sk.SK_ERR_INVALID_ARG


LOW_EPS = [(1e-2, 0.0), (1e-2, 1.0), (3e-3, 0.0), (3e-3, 1.0), (1e-3, 0.0), (1e-3, 1.0), (3e-4, 1.0)]


@pytest.mark.parametrize("eps,eps_start", LOW_EPS)
def test_low_eps_iterations_against_float64(sk, eps, eps_start):
    """Iterations to a marginal tolerance at low eps, float32 GPU against the
    float64 oracle under the same schedule and stopping rule (the mixture
    geometry of the 10k configuration at n = 256, m = 293, alternating, a check
    every 10 iterations). The error the GPU measures from float32 potentials
    carries an absolute uncertainty of about its floor, 2^-24 max|f| / eps (the
    weights sum to 1), so near the tolerance the two runs may stop one check
    apart. Where the floor is at most half the tolerance, the GPU stops within
    one check of the oracle; where it is not (eps = 3e-4 here), the float32
    measurement decides late by up to a tenth of the run. Either way the pair
    it returns meets the tolerance by the oracle's own marginals up to twice
    that floor."""
    from dataclasses import replace
    w = replace(W.CASES[2], eps=eps, mode="alternating").scaled(256, 293)
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    tol, every, cap = 1e-4, 10, 20000
    f, g, _, n_g, e_g = sk.solve_tol(x, y, a, b, eps, tol, cap, "alternating", every, eps_start=eps_start)
    fo, go, n_o, e_o = oracle.solve_tol(inp.x64(), inp.y64(), inp.a, inp.b, eps, tol, cap, "alternating", every,
                                        eps_start)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    r, c = oracle.marginals(inp.x64(), inp.y64(), inp.a, inp.b, t(f), t(g), eps)
    e_ret = np.abs(r - inp.a).sum() + np.abs(c - inp.b).sum()
    floor = 2.0 ** -24 * np.abs(t(f)).max() / eps
    say(f"low eps={eps:g} eps_start={eps_start:g}: float64 {n_o} iterations (err {e_o:.3e}), "
        f"GPU {n_g} (err {e_g:.3e}); returned pair's float64 error {e_ret:.3e}; float32 floor ~{floor:.1e}")
    assert n_o < cap and e_o <= tol and e_g <= tol
    if floor <= 0.5 * tol:
        assert abs(n_g - n_o) <= every
    else:
        assert abs(n_g - n_o) <= every + 0.1 * n_o
    assert e_ret <= tol + 2.0 * floor


def test_solve_tol_with_eps_scaling(sk):
    """eps-scaling (one iteration per halving from eps_start) then the tolerance
    phase at eps: the returned pair meets the tolerance by the oracle's marginals."""
    w = W.CASES[6].scaled(900, 800)
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    tol = 1e-4
    _, _, _, plain, _ = sk.solve_tol(x, y, a, b, w.eps, tol, 5000, check_every=10)
    f, g, _, done, err = sk.solve_tol(x, y, a, b, w.eps, tol, 5000, check_every=10, eps_start=2.0)
    t = lambda v: v.cpu().numpy().astype(np.float64)  # noqa: E731
    r, c = oracle.marginals(inp.x64(), inp.y64(), inp.a, inp.b, t(f), t(g), w.eps)
    ref = np.abs(r - inp.a).sum() + np.abs(c - inp.b).sum()
    say(f"eps-scaling from 2.0 to {w.eps}: {done} iterations (without: {plain}); err {err:.2e}, oracle {ref:.2e}")
    assert done < 5000 and err <= tol and ref <= tol


@pytest.mark.parametrize("key", [3, 2])
def test_hvp_and_hadamard_properties_at_full_size(sk, key):
    """At full size (no dense oracle): the Hessian is symmetric, <U, H V> =
    <V, H U>, and the Hadamard-weighted application with W = 1 1^T is the plain
    application bit for bit."""
    w = W.CASES[key]
    say(f"full-size HVP symmetry / Hadamard identity cfg={key} n={w.n} m={w.m} d={w.d}")
    inp = W.make_inputs(w, k=16)
    x, y, a, b = dev(inp)
    f, g, _ = sk.solve(x, y, a, b, w.eps, w.iters, "alternating")
    gen = torch.Generator(device=DEV).manual_seed(key)
    U = torch.randn(w.n, w.d, generator=gen, device=DEV)
    V = torch.randn(w.n, w.d, generator=gen, device=DEV)
    HV, iv, rv = sk.ot_hvp_x(x, y, a, b, f, g, w.eps, V)
    HU, iu, ru = sk.ot_hvp_x(x, y, a, b, f, g, w.eps, U)
    l, r = float((U.double() * HV.double()).sum()), float((V.double() * HU.double()).sum())
    scale = float(U.double().norm() * HV.double().norm())
    say(f"  CG {iv}/{iu} iterations (residuals {rv:.1e}, {ru:.1e}); <U,HV>={l:.6e} <V,HU>={r:.6e}")
    assert abs(l - r) <= 1e-4 * scale
    Vv = torch.from_numpy(inp.V).to(DEV)
    ones_n, ones_m = torch.ones(w.n, 1, device=DEV), torch.ones(w.m, 1, device=DEV)
    plain = sk.transport_apply(x, y, a, b, f, g, w.eps, Vv)
    had = sk.transport_apply_hadamard(x, y, a, b, f, g, w.eps, ones_n, ones_m, Vv)
    assert torch.equal(plain, had)


def _newton_reference():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_newton.json")
    with open(path) as fh:
        return json.load(fh)


@pytest.mark.parametrize("case", range(len(NC.CASES)))
def test_newton_matches_float64_newton(sk, case):
    """Newton-CG on x -> OT_eps(mu_x, nu) against the float64 oracle's Newton-CG
    (same algorithm; dense Moore-Penrose Hessian-vector products; stored by
    tests/golden/make_oracle_newton.py) from the same float32 start: the same
    cost after the first step, and the same stationary point. Later iterates
    may part slightly: the inner CG stops on a threshold (the forcing term),
    which float32 and float64 residuals can cross at different inner steps."""
    ref = _newton_reference()
    assert ref["oracle_sha256"] == NC.oracle_digest(), "oracle changed: the stored Newton references are stale"
    seed, n, m, d, eps = NC.CASES[case]
    r = ref["cases"][case]
    assert (r["seed"], r["n"], r["m"], r["d"], r["eps"]) == (seed, n, m, d, eps)
    x0, y, a, b = NC.inputs(seed, n, m, d)
    say(f"newton seed={seed} n={n} m={m} d={d} eps={eps}")
    t = lambda v: torch.from_numpy(v).to(DEV)  # noqa: E731
    # the marginal tolerance of each solve stays above the float32 floor of the
    # measured error (2^-24 max|f| / eps, about 1e-6 here)
    x, costs, norms, steps = sk.ot_newton_x(t(x0), t(y), t(a), t(b), eps, newton_iters=NC.NEWTON_ITERS, sk_tol=1e-5,
                                            sk_max_iters=4000, grad_tol=NC.GRAD_TOL)
    costs_o, norms_o = np.array(r["costs"]), np.array(r["grad_norms"])
    xo = np.array(r["x"]).reshape(n, d)
    say(f"  GPU {steps} steps, costs {np.array(costs)}, |grad| {np.array(norms)}")
    say(f"  float64 {r['steps']} steps, costs {costs_o}, |grad| {norms_o}")
    k = min(1, steps, r["steps"])
    assert np.allclose(costs[:k + 1], costs_o[:k + 1], rtol=1e-5, atol=0)
    assert norms[-1] <= 1e-4
    assert abs(costs[-1] - costs_o[-1]) <= 1e-5 * abs(costs_o[-1])
    assert np.abs(x.cpu().numpy() - xo).max() <= 2e-3


def test_newton_decreases_the_cost_at_full_shape(sk):
    """At n = m = 2000 (no dense reference): every step lowers the cost (Armijo)
    and the gradient norm falls by two orders of magnitude."""
    w = W.CASES[6].scaled(2000, 2000)
    inp = W.make_inputs(w)
    x, y, a, b = dev(inp)
    xs, costs, norms, steps = sk.ot_newton_x(x, y, a, b, 0.05, newton_iters=8, sk_tol=1e-4, sk_max_iters=4000)
    say(f"newton n=m=2000 d=3: {steps} steps, costs {np.array(costs)}, |grad| {np.array(norms)}")
    assert steps >= 3 and np.all(np.diff(costs) < 0)
    assert norms[-1] <= 1e-2 * norms[0]
