"""Streaming log-domain Sinkhorn on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libflashsk.so`` (include/flashsk.h).
It only marshals arguments: checks tensor devices, dtypes and shapes,
allocates outputs and the workspace with PyTorch, and passes raw device
pointers plus the current HIP stream. Every step of the computation runs in
the library's HIP kernels; there is no Python or CPU fallback, and importing
the package fails loudly if the shared library is missing.

    f, g, cost = solve(x, y, a, b, eps, iters, mode="alternating")
    f, g, cost, iters_done, err = solve_tol(x, y, a, b, eps, tol, max_iters)   # blocking
    out = transport_apply(x, y, a, b, f, g, eps, V)                  # P V
    out = transport_apply(x, y, a, b, f, g, eps, U, transpose=True)  # P^T U
    out = transport_apply_hadamard(x, y, a, b, f, g, eps, A, B, V)   # (P o A B^T) V
    grad = eot_grad_x(x, y, a, b, g, eps)
    HV, cg_iters, cg_resid = ot_hvp_x(x, y, a, b, f, g, eps, V)       # blocking
    x, costs, gnorms, steps = ot_newton_x(x0, y, a, b, eps)          # Newton-CG, blocking
    S, ga, gb, gx, gy = sinkhorn_divergence(x, y, a, b, eps, iters)  # debiased

x, y: (n, d) and (m, d) float32 or bfloat16 CUDA tensors; a, b, f, g, V, U:
float32. Plans, potentials and costs follow the conventions of flashsk.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflashsk.so")

SK_OK, SK_ERR_INVALID_ARG, SK_ERR_UNSUPPORTED, SK_ERR_WORKSPACE, SK_ERR_HIP = 0, -1, -2, -3, -4
SK_F32, SK_BF16 = 0, 1
SK_ALTERNATING, SK_SYMMETRIC = 0, 1
SK_WARM_START, SK_NO_CENTER, SK_CHECK_FINITE = 1, 2, 4
SK_OP_SOLVE, SK_OP_APPLY, SK_OP_GRAD, SK_OP_DIVERGENCE, SK_OP_APPLY_HADAMARD, SK_OP_SOLVE_TOL, SK_OP_HVP, SK_OP_NEWTON = range(8)

_ERR_NAMES = {SK_ERR_INVALID_ARG: "SK_ERR_INVALID_ARG", SK_ERR_UNSUPPORTED: "SK_ERR_UNSUPPORTED",
              SK_ERR_WORKSPACE: "SK_ERR_WORKSPACE", SK_ERR_HIP: "SK_ERR_HIP"}


class SinkhornError(RuntimeError):
    """A non-zero return code of the C ABI."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


def _load_library() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python streaming_sinkhorn_solver_log_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, U32, D, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                               ctypes.c_double, ctypes.c_size_t)
    INT = ctypes.c_int
    lib.sk_sinkhorn_solve.argtypes = [P, P, INT, I64, I64, I64, P, P, D, I32, INT, U32, P, P, P, P, SZ, P]
    lib.sk_sinkhorn_solve.restype = INT
    lib.sk_transport_apply.argtypes = [P, P, INT, I64, I64, I64, P, P, P, P, D, INT, P, I64, P, P, SZ, P]
    lib.sk_transport_apply.restype = INT
    lib.sk_eot_grad_x.argtypes = [P, P, INT, I64, I64, I64, P, P, P, D, P, P, SZ, P]
    lib.sk_eot_grad_x.restype = INT
    lib.sk_sinkhorn_divergence.argtypes = [P, P, INT, I64, I64, I64, P, P, D, I32, INT, U32, P, P, P, P, P, P,
                                           SZ, P]
    lib.sk_sinkhorn_divergence.restype = INT
    lib.sk_transport_apply_hadamard.argtypes = [P, P, INT, I64, I64, I64, P, P, P, P, D, INT, P, P, I64, P, I64,
                                                P, P, SZ, P]
    lib.sk_transport_apply_hadamard.restype = INT
    lib.sk_sinkhorn_solve_tol.argtypes = [P, P, INT, I64, I64, I64, P, P, D, D, I32, INT, U32, D, I32, P, P, P, P,
                                          P, P, SZ, P]
    lib.sk_sinkhorn_solve_tol.restype = INT
    lib.sk_ot_hvp_x.argtypes = [P, P, INT, I64, I64, I64, P, P, P, P, D, P, P, D, I32, P, P, P, SZ, P]
    lib.sk_ot_hvp_x.restype = INT
    lib.sk_ot_newton_x.argtypes = [P, P, I64, I64, I64, P, P, D, D, I32, I32, D, I32, P, P, P, P, P, SZ, P]
    lib.sk_ot_newton_x.restype = INT
    lib.sk_sinkhorn_solve_noalloc.argtypes = [P, P, INT, I64, I64, I64, P, P, D, I32, INT, U32, P, P, P, P]
    lib.sk_sinkhorn_solve_noalloc.restype = INT
    lib.sk_noalloc_scratch_bytes.argtypes = []
    lib.sk_noalloc_scratch_bytes.restype = SZ
    lib.sk_workspace_bytes.argtypes = [INT, INT, I64, I64, I64, I64]
    lib.sk_workspace_bytes.restype = SZ
    lib.sk_last_error.argtypes = []
    lib.sk_last_error.restype = ctypes.c_char_p
    lib.sk_version.argtypes = []
    lib.sk_version.restype = INT
    return lib


_lib = _load_library()
EXPORTS = ("sk_sinkhorn_solve", "sk_sinkhorn_solve_tol", "sk_transport_apply", "sk_transport_apply_hadamard", "sk_eot_grad_x",
           "sk_ot_hvp_x", "sk_ot_newton_x", "sk_sinkhorn_divergence", "sk_sinkhorn_solve_noalloc",
           "sk_noalloc_scratch_bytes",
           "sk_workspace_bytes", "sk_last_error", "sk_version")


def library() -> ctypes.CDLL:
    return _lib


def _check(rc: int) -> None:
    if rc != SK_OK:
        raise SinkhornError(rc, _lib.sk_last_error().decode(errors="replace"))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SK_F32
    if t.dtype == torch.bfloat16:
        return SK_BF16
    raise TypeError(f"points must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _vec(t: torch.Tensor, n: int, name: str, device) -> torch.Tensor:
    if t.dtype != torch.float32 or t.device != device or t.shape != (n,) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape ({n},) on {device}")
    return t


def _points(x: torch.Tensor, y: torch.Tensor):
    if not (x.is_cuda and y.is_cuda):
        raise ValueError("x and y must be GPU tensors")
    if x.dim() != 2 or y.dim() != 2 or x.shape[1] != y.shape[1]:
        raise ValueError("x must be (n, d) and y (m, d) with the same d")
    if x.dtype != y.dtype or x.device != y.device:
        raise ValueError("x and y must share dtype and device")
    if not (x.is_contiguous() and y.is_contiguous()):
        raise ValueError("x and y must be contiguous")
    return x.shape[0], y.shape[0], x.shape[1], _dtype_code(x)


def workspace_bytes(op: int, dtype: int, n: int, m: int, d: int, k: int = 0) -> int:
    return int(_lib.sk_workspace_bytes(op, dtype, n, m, d, k))


def _workspace(op, dtype, n, m, d, k, device, ws):
    """A 256-byte aligned region of at least the required size. With ws=None a
    new uint8 tensor is allocated on the current stream, which the library's
    launches use too, so the caching allocator cannot hand it to other work
    before they finish. A caller's workspace is used as given: it must be a
    contiguous uint8 tensor on the device holding the required bytes after
    its first 256-byte aligned address, else ValueError."""
    need = workspace_bytes(op, dtype, n, m, d, k)
    if need == 0:
        need = 256  # invalid sizes: the library reports the reason
    if ws is None:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=device)
    elif ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    elif ws.numel() < need + (-ws.data_ptr()) % 256:
        raise ValueError(f"workspace holds {ws.numel()} bytes; this call needs {need} bytes after a "
                         f"256-byte aligned start ({need + (-ws.data_ptr()) % 256} from this tensor's start)")
    off = (-ws.data_ptr()) % 256
    return ws, ws.data_ptr() + off, ws.numel() - off


def solve(x, y, a, b, eps: float, iters: int, mode: str = "alternating", f0=None, g0=None,
          center: bool = True, workspace=None, check_finite: bool = False):
    """Fixed-budget Sinkhorn; returns (f, g, cost) with cost a 0-d float64 tensor.
    check_finite: screen x, y, a, b (and f0, g0) on the device first and raise
    SinkhornError on a NaN, an infinity or a bad weight (waits for the stream)."""
    n, m, d, dt = _points(x, y)
    dev = x.device
    _vec(a, n, "a", dev)
    _vec(b, m, "b", dev)
    mode_code = {"alternating": SK_ALTERNATING, "symmetric": SK_SYMMETRIC}[mode]
    flags = (0 if center else SK_NO_CENTER) | (SK_CHECK_FINITE if check_finite else 0)
    if (f0 is None) != (g0 is None):
        raise ValueError("give both f0 and g0 for a warm start, or neither")
    if f0 is not None:
        f = _vec(f0, n, "f0", dev).clone()
        g = _vec(g0, m, "g0", dev).clone()
        flags |= SK_WARM_START
    else:
        f = torch.empty(n, dtype=torch.float32, device=dev)
        g = torch.empty(m, dtype=torch.float32, device=dev)
    cost = torch.empty((), dtype=torch.float64, device=dev)
    ws, wptr, wbytes = _workspace(SK_OP_SOLVE, dt, n, m, d, 0, dev, workspace)
    with torch.cuda.device(dev):  # the library's HIP calls act on the current device
        _check(_lib.sk_sinkhorn_solve(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), float(eps),
                                      int(iters), mode_code, flags, _ptr(f), _ptr(g), _ptr(cost),
                                      ctypes.c_void_p(wptr), wbytes, _stream(dev)))
    return f, g, cost


def solve_noalloc(x, y, a, b, eps: float, iters: int, mode: str = "alternating", f0=None, g0=None,
                  center: bool = True):
    """solve() on the library's own per-GPU scratch (sk_sinkhorn_solve_noalloc):
    no workspace is allocated or passed. Outputs are still new tensors here;
    callers that cannot allocate call the C entry point with their own."""
    n, m, d, dt = _points(x, y)
    dev = x.device
    _vec(a, n, "a", dev)
    _vec(b, m, "b", dev)
    mode_code = {"alternating": SK_ALTERNATING, "symmetric": SK_SYMMETRIC}[mode]
    flags = 0 if center else SK_NO_CENTER
    if (f0 is None) != (g0 is None):
        raise ValueError("give both f0 and g0 for a warm start, or neither")
    if f0 is not None:
        f = _vec(f0, n, "f0", dev).clone()
        g = _vec(g0, m, "g0", dev).clone()
        flags |= SK_WARM_START
    else:
        f = torch.empty(n, dtype=torch.float32, device=dev)
        g = torch.empty(m, dtype=torch.float32, device=dev)
    cost = torch.empty((), dtype=torch.float64, device=dev)
    with torch.cuda.device(dev):
        _check(_lib.sk_sinkhorn_solve_noalloc(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), float(eps),
                                              int(iters), mode_code, flags, _ptr(f), _ptr(g), _ptr(cost),
                                              _stream(dev)))
    return f, g, cost


def transport_apply(x, y, a, b, f, g, eps: float, V, transpose: bool = False, workspace=None):
    """P V (V: m x k), or P^T V (V: n x k) with transpose=True."""
    n, m, d, dt = _points(x, y)
    dev = x.device
    for t, cnt, name in ((a, n, "a"), (b, m, "b"), (f, n, "f"), (g, m, "g")):
        _vec(t, cnt, name, dev)
    squeeze = V.dim() == 1
    V2 = V[:, None] if squeeze else V
    rows_in = n if transpose else m
    if V2.dtype != torch.float32 or V2.device != dev or V2.dim() != 2 or V2.shape[0] != rows_in:
        raise ValueError(f"V must be float32 of shape ({rows_in}, k) on {dev}")
    V2 = V2.contiguous()
    k = V2.shape[1]
    out = torch.empty((m if transpose else n, k), dtype=torch.float32, device=dev)
    ws, wptr, wbytes = _workspace(SK_OP_APPLY, dt, n, m, d, k, dev, workspace)
    with torch.cuda.device(dev):
        _check(_lib.sk_transport_apply(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), _ptr(f), _ptr(g),
                                       float(eps), int(bool(transpose)), _ptr(V2), k, _ptr(out),
                                       ctypes.c_void_p(wptr), wbytes, _stream(dev)))
    return out[:, 0] if squeeze else out


def eot_grad_x(x, y, a, b, g, eps: float, workspace=None):
    """Barycentric-projection gradient of the EOT cost with respect to x (n x d)."""
    n, m, d, dt = _points(x, y)
    dev = x.device
    for t, cnt, name in ((a, n, "a"), (b, m, "b"), (g, m, "g")):
        _vec(t, cnt, name, dev)
    out = torch.empty((n, d), dtype=torch.float32, device=dev)
    ws, wptr, wbytes = _workspace(SK_OP_GRAD, dt, n, m, d, 0, dev, workspace)
    with torch.cuda.device(dev):
        _check(_lib.sk_eot_grad_x(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), _ptr(g), float(eps),
                                  _ptr(out), ctypes.c_void_p(wptr), wbytes, _stream(dev)))
    return out


def sinkhorn_divergence(x, y, a, b, eps: float, iters: int, mode: str = "alternating", grads: bool = True,
                        center: bool = True, workspace=None, check_finite: bool = False):
    """Debiased Sinkhorn divergence S = OT(a,b) - OT(a,a)/2 - OT(b,b)/2 (flashsk.h).

    Returns (S, grad_a, grad_b, grad_x, grad_y): S a 0-d float64 tensor, the
    gradients float32 (None when grads=False). check_finite: screen x, y, a, b
    on the device first (as for solve).
    """
    n, m, d, dt = _points(x, y)
    dev = x.device
    _vec(a, n, "a", dev)
    _vec(b, m, "b", dev)
    mode_code = {"alternating": SK_ALTERNATING, "symmetric": SK_SYMMETRIC}[mode]
    flags = (0 if center else SK_NO_CENTER) | (SK_CHECK_FINITE if check_finite else 0)
    S = torch.empty((), dtype=torch.float64, device=dev)
    ga = gb = gx = gy = None
    if grads:
        ga = torch.empty(n, dtype=torch.float32, device=dev)
        gb = torch.empty(m, dtype=torch.float32, device=dev)
        gx = torch.empty((n, d), dtype=torch.float32, device=dev)
        gy = torch.empty((m, d), dtype=torch.float32, device=dev)
    ws, wptr, wbytes = _workspace(SK_OP_DIVERGENCE, dt, n, m, d, 0, dev, workspace)
    with torch.cuda.device(dev):
        _check(_lib.sk_sinkhorn_divergence(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), float(eps),
                                           int(iters), mode_code, flags, _ptr(S), _ptr(ga), _ptr(gb),
                                           _ptr(gx), _ptr(gy), ctypes.c_void_p(wptr), wbytes, _stream(dev)))
    return S, ga, gb, gx, gy


def transport_apply_hadamard(x, y, a, b, f, g, eps: float, A, B, V, transpose: bool = False, workspace=None):
    """(P o W) V with W = A B^T (A: n x r, B: m x r; V: m x k), or (P o W)^T V
    (V: n x k) with transpose=True."""
    n, m, d, dt = _points(x, y)
    dev = x.device
    for t, cnt, name in ((a, n, "a"), (b, m, "b"), (f, n, "f"), (g, m, "g")):
        _vec(t, cnt, name, dev)
    A2 = A[:, None] if A.dim() == 1 else A
    B2 = B[:, None] if B.dim() == 1 else B
    if (A2.dtype != torch.float32 or B2.dtype != torch.float32 or A2.device != dev or B2.device != dev
            or A2.dim() != 2 or B2.dim() != 2 or A2.shape[0] != n or B2.shape[0] != m
            or A2.shape[1] != B2.shape[1]):
        raise ValueError(f"A and B must be float32 (n, r) and (m, r) on {dev} with the same r")
    A2, B2 = A2.contiguous(), B2.contiguous()
    squeeze = V.dim() == 1
    V2 = V[:, None] if squeeze else V
    rows_in = n if transpose else m
    if V2.dtype != torch.float32 or V2.device != dev or V2.dim() != 2 or V2.shape[0] != rows_in:
        raise ValueError(f"V must be float32 of shape ({rows_in}, k) on {dev}")
    V2 = V2.contiguous()
    k, r = V2.shape[1], A2.shape[1]
    out = torch.empty((m if transpose else n, k), dtype=torch.float32, device=dev)
    ws, wptr, wbytes = _workspace(SK_OP_APPLY_HADAMARD, dt, n, m, d, k, dev, workspace)
    with torch.cuda.device(dev):
        _check(_lib.sk_transport_apply_hadamard(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), _ptr(f), _ptr(g),
                                                float(eps), int(bool(transpose)), _ptr(A2), _ptr(B2), r, _ptr(V2),
                                                k, _ptr(out), ctypes.c_void_p(wptr), wbytes, _stream(dev)))
    return out[:, 0] if squeeze else out


def solve_tol(x, y, a, b, eps: float, tol: float, max_iters: int, mode: str = "alternating",
              check_every: int = 10, f0=None, g0=None, center: bool = True, eps_start: float = 0.0,
              workspace=None, check_finite: bool = False):
    """Sinkhorn until the marginal error ||P1 - a||_1 + ||P^T 1 - b||_1 of the
    pair checked every `check_every` iterations is <= tol (or max_iters), after
    an optional eps-scaling from eps_start (one iteration per halving).
    Blocking. Returns (f, g, cost, iters_done, err)."""
    n, m, d, dt = _points(x, y)
    dev = x.device
    _vec(a, n, "a", dev)
    _vec(b, m, "b", dev)
    mode_code = {"alternating": SK_ALTERNATING, "symmetric": SK_SYMMETRIC}[mode]
    flags = (0 if center else SK_NO_CENTER) | (SK_CHECK_FINITE if check_finite else 0)
    if (f0 is None) != (g0 is None):
        raise ValueError("give both f0 and g0 for a warm start, or neither")
    if f0 is not None:
        f = _vec(f0, n, "f0", dev).clone()
        g = _vec(g0, m, "g0", dev).clone()
        flags |= SK_WARM_START
    else:
        f = torch.empty(n, dtype=torch.float32, device=dev)
        g = torch.empty(m, dtype=torch.float32, device=dev)
    cost = torch.empty((), dtype=torch.float64, device=dev)
    done = ctypes.c_int32(0)
    err = ctypes.c_double(0.0)
    ws, wptr, wbytes = _workspace(SK_OP_SOLVE_TOL, dt, n, m, d, 0, dev, workspace)
    with torch.cuda.device(dev):
        _check(_lib.sk_sinkhorn_solve_tol(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), float(eps),
                                          float(eps_start), int(max_iters), mode_code, flags, float(tol),
                                          int(check_every),
                                          _ptr(f), _ptr(g), _ptr(cost), ctypes.byref(done), ctypes.byref(err),
                                          ctypes.c_void_p(wptr), wbytes, _stream(dev)))
    return f, g, cost, done.value, err.value


def ot_hvp_x(x, y, a, b, f, g, eps: float, V, cg_tol: float = 1e-6, cg_max_iters: int = 500, workspace=None):
    """Hessian of OT_eps in x applied to V (n x d) at the pair (f, g), matrix-free.
    Blocking. Returns (HV, cg_iters, cg_relative_residual)."""
    n, m, d, dt = _points(x, y)
    dev = x.device
    for t, cnt, name in ((a, n, "a"), (b, m, "b"), (f, n, "f"), (g, m, "g")):
        _vec(t, cnt, name, dev)
    if V.dtype != torch.float32 or V.device != dev or tuple(V.shape) != (n, d):
        raise ValueError(f"V must be float32 of shape ({n}, {d}) on {dev}")
    V = V.contiguous()
    out = torch.empty((n, d), dtype=torch.float32, device=dev)
    iters = ctypes.c_int32(0)
    resid = ctypes.c_double(0.0)
    ws, wptr, wbytes = _workspace(SK_OP_HVP, dt, n, m, d, 0, dev, workspace)
    with torch.cuda.device(dev):
        _check(_lib.sk_ot_hvp_x(_ptr(x), _ptr(y), dt, n, m, d, _ptr(a), _ptr(b), _ptr(f), _ptr(g), float(eps),
                                _ptr(V), _ptr(out), float(cg_tol), int(cg_max_iters), ctypes.byref(iters),
                                ctypes.byref(resid), ctypes.c_void_p(wptr), wbytes, _stream(dev)))
    return out, iters.value, resid.value


def ot_newton_x(x0, y, a, b, eps: float, newton_iters: int = 10, sk_tol: float = 1e-5, sk_max_iters: int = 20000,
                grad_tol: float = 0.0, cg_max_iters: int = 100, workspace=None):
    """Line-search Newton-CG on the points x of the first measure, minimizing
    OT_eps(sum_i a_i delta_{x_i}, sum_j b_j delta_{y_j}) (flashsk.h,
    sk_ot_newton_x); x0 (n, d) and y (m, d) float32. Blocking. Returns
    (x, costs, grad_norms, steps): the last iterate, and float64 arrays of
    the cost and gradient norm at iterates 0..steps."""
    n, m, d, dt = _points(x0, y)
    if dt != SK_F32:
        raise TypeError("Newton-CG takes float32 points")
    dev = x0.device
    _vec(a, n, "a", dev)
    _vec(b, m, "b", dev)
    x = torch.empty_like(x0)
    costs = (ctypes.c_double * (newton_iters + 1))()
    norms = (ctypes.c_double * (newton_iters + 1))()
    steps = ctypes.c_int32(0)
    ws, wptr, wbytes = _workspace(SK_OP_NEWTON, dt, n, m, d, 0, dev, workspace)
    with torch.cuda.device(dev):
        _check(_lib.sk_ot_newton_x(_ptr(x0), _ptr(y), n, m, d, _ptr(a), _ptr(b), float(eps), float(sk_tol),
                                   int(sk_max_iters), int(newton_iters), float(grad_tol), int(cg_max_iters),
                                   _ptr(x), costs, norms, ctypes.byref(steps), ctypes.c_void_p(wptr), wbytes,
                                   _stream(dev)))
    k = steps.value
    return x, [costs[i] for i in range(k + 1)], [norms[i] for i in range(k + 1)], k
