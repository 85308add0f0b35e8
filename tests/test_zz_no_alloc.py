"""The allocation-free solve (sk_sinkhorn_solve_noalloc) against the solve
with a caller workspace, through the C ABI: two calls in a row on the same
device scratch, the second smaller than the first, each bitwise equal to
sk_sinkhorn_solve on the same inputs; sizes beyond the scratch are refused
before anything is enqueued."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(f"[noalloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sk():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import streaming_sinkhorn_solver_log_amd as sk
    return sk


def _entry(sk):
    fn = sk.library().sk_sinkhorn_solve_noalloc
    P, I64, I32, U32, D, INT = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_double,
                                ctypes.c_int)
    fn.argtypes = [P, P, INT, I64, I64, I64, P, P, D, I32, INT, U32, P, P, P, P]
    fn.restype = INT
    return fn


def _dev(inp):
    if inp.w.dtype == "bf16":
        x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).to(DEV)
        y = torch.from_numpy(inp.y.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        x, y = torch.from_numpy(inp.x).to(DEV), torch.from_numpy(inp.y).to(DEV)
    return x, y, torch.from_numpy(inp.a).to(DEV), torch.from_numpy(inp.b).to(DEV)


def _noalloc(sk, fn, x, y, a, b, eps, iters, mode):
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    dt = sk.SK_BF16 if x.dtype == torch.bfloat16 else sk.SK_F32
    f = torch.full((n,), float("nan"), device=DEV)
    g = torch.full((m,), float("nan"), device=DEV)
    cost = torch.full((), float("nan"), dtype=torch.float64, device=DEV)
    code = {"alternating": sk.SK_ALTERNATING, "symmetric": sk.SK_SYMMETRIC}[mode]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fn(x.data_ptr(), y.data_ptr(), dt, n, m, d, a.data_ptr(), b.data_ptr(), eps, iters, code, 0,
            f.data_ptr(), g.data_ptr(), cost.data_ptr(), stream)
    return rc, f, g, cost


# (config key, n, m, iters, mode): each pair is two calls in a row, the second smaller
PAIRS = [
    [(3, 50_000, 50_000, 20, "alternating"), (3, 7_000, 5_500, 9, "alternating")],  # bf16 d = 64, full size first
    [(6, 30_000, 26_000, 12, "symmetric"), (1, 900, 700, 15, "alternating")],      # float32 d = 3, both schedules
    [(7, 3_000, 2_500, 5, "alternating"), (7, 800, 600, 5, "symmetric")],          # bf16 d = 512, GEMM-tiled
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_solve_matches_workspace_solve(sk, pair):
    fn = _entry(sk)
    for key, n, m, iters, mode in PAIRS[pair]:
        w = W.CASES[key].scaled(n, m, iters)
        say(f"cfg={key} n={n} m={m} d={w.d} {w.dtype} iters={iters} {mode}")
        inp = W.make_inputs(w)
        x, y, a, b = _dev(inp)
        rc, f, g, cost = _noalloc(sk, fn, x, y, a, b, w.eps, iters, mode)
        assert rc == 0, sk.library().sk_last_error()
        fr, gr, cr = sk.solve(x, y, a, b, w.eps, iters, mode)
        torch.cuda.synchronize()
        assert torch.equal(f, fr) and torch.equal(g, gr) and torch.equal(cost, cr)


def test_noalloc_refuses_sizes_beyond_its_scratch(sk):
    fn = _entry(sk)
    lib = sk.library()
    lib.sk_noalloc_scratch_bytes.restype = ctypes.c_size_t
    limit = lib.sk_noalloc_scratch_bytes()
    w = W.CASES[4].scaled(20_000, 20_000, 2)  # float32 d = 512: about 477 MiB of scratch
    assert sk.workspace_bytes(sk.SK_OP_SOLVE, sk.SK_F32, w.n, w.m, w.d) > limit
    inp = W.make_inputs(w)
    x, y, a, b = _dev(inp)
    rc, f, g, cost = _noalloc(sk, fn, x, y, a, b, w.eps, 2, "alternating")
    torch.cuda.synchronize()
    assert rc == sk.SK_ERR_UNSUPPORTED
    assert b"scratch" in lib.sk_last_error()
    assert torch.isnan(f).all() and torch.isnan(g).all() and torch.isnan(cost)
