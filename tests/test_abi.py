"""The C-ABI library loads, exports every symbol include/flashsk.h declares, and
rejects invalid arguments on the host before anything reaches a GPU.

No test here makes a compute call: every call below fails validation, which
happens before the first HIP call, so the suite runs on machines without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashsk.h")
# FLASHSK_ABI_LIB: another build of the same library (the host-sanitized one,
# tests/test_sanitized_abi.py)
LIB = os.environ.get("FLASHSK_ABI_LIB") or os.path.join(ROOT, "streaming_sinkhorn_solver_log_amd", "libflashsk.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sk_[a-z_]+)\s*\(", src)))


def _header_int(name):
    m = re.search(r"#define\s+%s\s+\(?(-?\w+)u?\)?" % name, open(HEADER).read())
    return int(m.group(1).rstrip("u"), 0)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libflashsk.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    P, I64, I32, U32, D, SZ, INT = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                                    ctypes.c_double, ctypes.c_size_t, ctypes.c_int)
    L.sk_sinkhorn_solve.argtypes = [P, P, INT, I64, I64, I64, P, P, D, I32, INT, U32, P, P, P, P, SZ, P]
    L.sk_transport_apply.argtypes = [P, P, INT, I64, I64, I64, P, P, P, P, D, INT, P, I64, P, P, SZ, P]
    L.sk_eot_grad_x.argtypes = [P, P, INT, I64, I64, I64, P, P, P, D, P, P, SZ, P]
    L.sk_sinkhorn_divergence.argtypes = [P, P, INT, I64, I64, I64, P, P, D, I32, INT, U32, P, P, P, P, P, P,
                                         SZ, P]
    L.sk_sinkhorn_solve_tol.argtypes = [P, P, INT, I64, I64, I64, P, P, D, D, I32, INT, U32, D, I32, P, P, P, P, P,
                                        P, SZ, P]
    L.sk_ot_hvp_x.argtypes = [P, P, INT, I64, I64, I64, P, P, P, P, D, P, P, D, I32, P, P, P, SZ, P]
    L.sk_transport_apply_hadamard.argtypes = [P, P, INT, I64, I64, I64, P, P, P, P, D, INT, P, P, I64, P, I64, P,
                                              P, SZ, P]
    L.sk_workspace_bytes.argtypes = [INT, INT, I64, I64, I64, I64]
    L.sk_workspace_bytes.restype = SZ
    L.sk_last_error.restype = ctypes.c_char_p
    return L


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"sk_sinkhorn_solve", "sk_transport_apply", "sk_eot_grad_x",
                          "sk_sinkhorn_divergence", "sk_transport_apply_hadamard", "sk_sinkhorn_solve_tol",
                          "sk_ot_hvp_x", "sk_workspace_bytes",
                          "sk_last_error", "sk_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.sk_version() == _header_int("SK_VERSION")
    assert lib.sk_last_error() is not None


def test_workspace_sizes(lib):
    solve, apply, grad = _header_int("SK_OP_SOLVE"), _header_int("SK_OP_APPLY"), _header_int("SK_OP_GRAD")
    for d in (1, 3, 16):
        for n, m in ((1, 1), (1024, 1024), (10_000, 777), (50_000, 50_000)):
            s = lib.sk_workspace_bytes(solve, 0, n, m, d, 0)
            assert s >= 4 * (n + m) * d
            assert lib.sk_workspace_bytes(apply, 0, n, m, d, 16) > 0
            assert lib.sk_workspace_bytes(grad, 0, n, m, d, 0) > 0
            # the divergence runs the three solves and four gradients in one workspace
            dv = lib.sk_workspace_bytes(_header_int("SK_OP_DIVERGENCE"), 0, n, m, d, 0)
            assert dv > max(s, lib.sk_workspace_bytes(solve, 0, n, n, d, 0),
                            lib.sk_workspace_bytes(solve, 0, m, m, d, 0))
            had = _header_int("SK_OP_APPLY_HADAMARD")
            assert lib.sk_workspace_bytes(had, 0, n, m, d, 16) >= lib.sk_workspace_bytes(apply, 0, n, m, d, 16)
            assert lib.sk_workspace_bytes(had, 0, n, m, d, 65) == 0
            assert lib.sk_workspace_bytes(_header_int("SK_OP_SOLVE_TOL"), 0, n, m, d, 0) > s
            assert lib.sk_workspace_bytes(_header_int("SK_OP_HVP"), 0, n, m, d, 0) > 0
    assert lib.sk_workspace_bytes(_header_int("SK_OP_HVP"), 0, 100, 100, 65, 0) > 0
    assert lib.sk_workspace_bytes(_header_int("SK_OP_HVP"), 0, 100, 100, 4097, 0) == 0
    assert lib.sk_workspace_bytes(solve, 0, 0, 5, 3, 0) == 0
    assert lib.sk_workspace_bytes(solve, 0, 5, 5, 0, 0) == 0
    assert lib.sk_workspace_bytes(apply, 0, 5, 5, 3, 0) == 0
    assert lib.sk_workspace_bytes(apply, 0, 5, 5, 3, 65) > 0
    assert lib.sk_workspace_bytes(apply, 0, 5, 5, 3, 4097) == 0
    assert lib.sk_workspace_bytes(99, 0, 5, 5, 3, 0) == 0


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _solve(lib, **kw):
    args = dict(x=FAKE, y=FAKE, dtype=0, n=10, m=12, d=3, a=FAKE, b=FAKE, eps=0.1, iters=3, mode=0,
                flags=0, f=FAKE, g=FAKE, cost=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.sk_sinkhorn_solve(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), "SK_ERR_INVALID_ARG"),
    (dict(b=None), "SK_ERR_INVALID_ARG"),
    (dict(f=None), "SK_ERR_INVALID_ARG"),
    (dict(cost=None), "SK_ERR_INVALID_ARG"),
    (dict(dtype=7), "SK_ERR_INVALID_ARG"),
    (dict(n=0), "SK_ERR_INVALID_ARG"),
    (dict(m=-3), "SK_ERR_INVALID_ARG"),
    (dict(d=0), "SK_ERR_INVALID_ARG"),
    (dict(eps=0.0), "SK_ERR_INVALID_ARG"),
    (dict(eps=-1.0), "SK_ERR_INVALID_ARG"),
    (dict(eps=float("nan")), "SK_ERR_INVALID_ARG"),
    (dict(eps=float("inf")), "SK_ERR_INVALID_ARG"),
    (dict(iters=-1), "SK_ERR_INVALID_ARG"),
    (dict(mode=2), "SK_ERR_INVALID_ARG"),
    (dict(flags=0x80), "SK_ERR_INVALID_ARG"),
    (dict(x=FAKE + 4), "SK_ERR_INVALID_ARG"),
    (dict(ws=None), "SK_ERR_WORKSPACE"),
    (dict(ws=FAKE + 64), "SK_ERR_WORKSPACE"),
    (dict(ws_bytes=16), "SK_ERR_WORKSPACE"),
    (dict(n=1 << 31), "SK_ERR_UNSUPPORTED"),
])
def test_solve_rejects_invalid_arguments(lib, kw, code):
    assert _solve(lib, **kw) == _header_int(code)
    assert len(lib.sk_last_error()) > 0


def test_apply_and_grad_reject_invalid_arguments(lib):
    inv, uns, wsp = _header_int("SK_ERR_INVALID_ARG"), _header_int("SK_ERR_UNSUPPORTED"), _header_int("SK_ERR_WORKSPACE")
    base = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, FAKE, FAKE, 0.1, 0, FAKE, 4, FAKE, FAKE, 1 << 30, None]
    for idx, val, code in [(11, 2, inv), (13, 0, inv), (13, 4097, uns), (12, None, inv), (14, None, inv),
                           (8, None, inv), (10, 0.0, inv), (15, None, wsp), (16, 8, wsp)]:
        args = list(base)
        args[idx] = val
        assert lib.sk_transport_apply(*args) == code, (idx, val)
    gbase = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 30, None]
    for idx, val, code in [(8, None, inv), (10, None, inv), (2, 5, inv), (9, -0.5, inv), (11, None, wsp)]:
        args = list(gbase)
        args[idx] = val
        assert lib.sk_eot_grad_x(*args) == code, (idx, val)


def test_divergence_rejects_invalid_arguments(lib):
    inv, wsp = _header_int("SK_ERR_INVALID_ARG"), _header_int("SK_ERR_WORKSPACE")
    warm = _header_int("SK_WARM_START")
    base = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, 0.1, 3, 0, 0, FAKE, None, None, None, None, FAKE, 1 << 30,
            None]
    for idx, val, code in [(0, None, inv), (6, None, inv), (8, 0.0, inv), (9, -1, inv), (10, 5, inv),
                           (11, warm, inv), (12, None, inv), (3, 0, inv), (17, None, wsp), (18, 64, wsp)]:
        args = list(base)
        args[idx] = val
        assert lib.sk_sinkhorn_divergence(*args) == code, (idx, val)
        assert len(lib.sk_last_error()) > 0


def test_hadamard_apply_rejects_invalid_arguments(lib):
    inv, uns, wsp = _header_int("SK_ERR_INVALID_ARG"), _header_int("SK_ERR_UNSUPPORTED"), _header_int("SK_ERR_WORKSPACE")
    base = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, FAKE, FAKE, 0.1, 0, FAKE, FAKE, 2, FAKE, 4, FAKE, FAKE, 1 << 30,
            None]
    for idx, val, code in [(12, None, inv), (13, None, inv), (14, 0, inv), (16, 0, inv), (16, 65, uns),
                           (11, 3, inv), (15, None, inv), (17, None, inv), (10, -1.0, inv), (18, None, wsp),
                           (19, 8, wsp)]:
        args = list(base)
        args[idx] = val
        assert lib.sk_transport_apply_hadamard(*args) == code, (idx, val)


def test_solve_tol_rejects_invalid_arguments(lib):
    inv, wsp = _header_int("SK_ERR_INVALID_ARG"), _header_int("SK_ERR_WORKSPACE")
    base = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, 0.1, 0.0, 100, 0, 0, 1e-4, 10, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, 1 << 30, None]
    for idx, val, code in [(10, 0, inv), (14, 0, inv), (13, -1.0, inv), (13, float("nan"), inv), (11, 3, inv),
                           (12, 0x40, inv), (18, None, inv), (19, None, inv), (15, None, inv), (20, None, wsp),
                           (21, 32, wsp), (8, 0.0, inv), (9, -1.0, inv), (9, float("inf"), inv)]:
        args = list(base)
        args[idx] = val
        assert lib.sk_sinkhorn_solve_tol(*args) == code, (idx, val)


def test_hvp_rejects_invalid_arguments(lib):
    inv, uns, wsp = _header_int("SK_ERR_INVALID_ARG"), _header_int("SK_ERR_UNSUPPORTED"), _header_int("SK_ERR_WORKSPACE")
    base = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, 1e-6, 100, FAKE, FAKE, FAKE, 1 << 30,
            None]
    for idx, val, code in [(8, None, inv), (11, None, inv), (12, None, inv), (13, 0.0, inv), (14, 0, inv),
                           (15, None, inv), (5, 4097, uns), (11, FAKE + 4, inv), (17, None, wsp), (18, 64, wsp)]:
        args = list(base)
        args[idx] = val
        assert lib.sk_ot_hvp_x(*args) == code, (idx, val)


def test_peaks_library_exports_measure_entry():
    """The unit-rate microbenchmark library bench.py --peaks loads exports its
    one entry point (loading it makes no GPU call)."""
    path = os.path.join(ROOT, "streaming_sinkhorn_solver_log_amd", "peaks", "libskpeaks.so")
    if not os.path.exists(path):
        pytest.skip("libskpeaks.so not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    assert hasattr(L, "skp_measure")


def test_check_finite_flag_matches_the_binding(lib):
    """SK_CHECK_FINITE is a known flag bit (unknown bits are still refused) and
    the Python binding uses the header's value."""
    flag = _header_int("SK_CHECK_FINITE")
    assert flag not in (_header_int("SK_WARM_START"), _header_int("SK_NO_CENTER"))
    src = open(os.path.join(ROOT, "streaming_sinkhorn_solver_log_amd", "__init__.py")).read()
    values = re.search(r"^SK_WARM_START, SK_NO_CENTER, SK_CHECK_FINITE = (.*)$", src, re.M).group(1)
    assert [int(v) for v in values.split(",")][2] == flag
    inv = _header_int("SK_ERR_INVALID_ARG")
    base = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, 0.1, 3, 0, flag | 0x80, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.sk_sinkhorn_solve(*base) == inv
    assert b"flag" in lib.sk_last_error()


def test_noalloc_solve_validates_before_any_device_call(lib):
    """The allocation-free solve refuses bad arguments, SK_CHECK_FINITE and sizes
    beyond its scratch on the host, before it looks up its device array."""
    P, I64, I32, U32, D, INT = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_double,
                                ctypes.c_int)
    fn = lib.sk_sinkhorn_solve_noalloc
    fn.argtypes = [P, P, INT, I64, I64, I64, P, P, D, I32, INT, U32, P, P, P, P]
    fn.restype = INT
    lib.sk_noalloc_scratch_bytes.restype = ctypes.c_size_t
    assert lib.sk_noalloc_scratch_bytes() == 64 << 20
    inv, uns = _header_int("SK_ERR_INVALID_ARG"), _header_int("SK_ERR_UNSUPPORTED")
    base = [FAKE, FAKE, 0, 10, 12, 3, FAKE, FAKE, 0.1, 3, 0, 0, FAKE, FAKE, FAKE, None]
    cases = [(0, None, inv), (8, -1.0, inv), (9, -1, inv), (10, 7, inv), (11, _header_int("SK_CHECK_FINITE"), inv),
             (12, None, inv), (3, 20_000, uns)]
    for idx, val, code in cases:
        args = list(base)
        args[idx] = val
        if idx == 3:  # float32 d = 512 at 20k x 20k needs far more than the scratch
            args[4], args[5] = 20_000, 512
        assert fn(*args) == code, (idx, val)
        assert len(lib.sk_last_error()) > 0


def test_newton_rejects_invalid_arguments(lib):
    P, I64, I32, D, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
    fn = lib.sk_ot_newton_x
    fn.argtypes = [P, P, I64, I64, I64, P, P, D, D, I32, I32, D, I32, P, P, P, P, P, SZ, P]
    fn.restype = ctypes.c_int
    inv, uns, wsp = _header_int("SK_ERR_INVALID_ARG"), _header_int("SK_ERR_UNSUPPORTED"), _header_int("SK_ERR_WORKSPACE")
    base = [FAKE, FAKE, 10, 12, 3, FAKE, FAKE, 0.1, 1e-5, 100, 5, 0.0, 50, FAKE, None, None, FAKE, FAKE, 1 << 30,
            None]
    for idx, val, code in [(0, None, inv), (13, None, inv), (16, None, inv), (8, 0.0, inv), (9, 0, inv),
                           (10, -1, inv), (11, -1.0, inv), (12, 0, inv), (4, 4097, uns), (7, 0.0, inv),
                           (17, None, wsp), (18, 64, wsp)]:
        args = list(base)
        args[idx] = val
        assert fn(*args) == code, (idx, val)
    assert lib.sk_workspace_bytes(_header_int("SK_OP_NEWTON"), 1, 10, 12, 3, 0) == 0  # float32 points only
    assert lib.sk_workspace_bytes(_header_int("SK_OP_NEWTON"), 0, 10, 12, 3, 0) > 0
