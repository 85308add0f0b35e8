#!/usr/bin/env python3
"""Benchmark of the streaming log-domain Sinkhorn hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
a fixed-budget solve (prep, `iters` iterations of an F and a G half-pass, the
cost), the barycentric gradient with respect to x, and the transport
applications P V and P^T U with k = 16. The reported value is Sinkhorn
iterations per second of the whole step (iterations per step / seconds per
step), so the gradient and applications count against it.

Default workload: n = m = 50,000, d = 64, bf16 points, Dirichlet weights,
eps = 0.1, 100 alternating iterations. The same JSON line carries the d = 3
point of the metric (n = m = 50,000, 8-Gaussian mixture, eps = 0.01,
100 alternating iterations) under "d3".

Timing: W untimed warm-up steps, then exactly K steps between two device
synchronizations. Inside the timed region every call is bracketed by HIP
events on the stream the library launches on (torch's current stream); the
average half-pass duration is (solve time - prep/cost time) / (2 iters).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "Sinkhorn iters/s at n=m=50k (d=3, d=64) + % of gfx950 roofline"
CU, CLK = 256, 2.4e9
# Non-packed fp32 VALU issue: 64 lanes per CU per clock; v_exp_f32 issues at
# half that rate (32 lanes per CU per clock), i.e. it takes two issue slots.
EXP_PEAK = CU * 32 * CLK            # exp2 evaluations per second
VALU_PEAK = CU * 64 * CLK           # fp32 VALU issue slots (lane-operations) per second
BF16_MFMA_PEAK = 2.5e15             # dense bf16 MFMA flop/s
F32_MFMA_PEAK = 157.3e12
HBM_PEAK = 8.0e12

WORKLOADS = {w.name: key for key, w in W.CASES.items()}

# HBM traffic of the half-pass kernels, from rocprofv3 FETCH_SIZE / WRITE_SIZE
# runs scaled by the same counters' reading for a device copy of known size
# (written by --summarize-counters). It is reported only while the kernel
# sources still hash to the digest the counters were taken with.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
_CSRC = os.path.join(ROOT, "streaming_sinkhorn_solver_log_amd", "csrc")
KERNEL_SOURCES = ["pass_mfma.hip", "sk_mfma_dev.h", "sk_mfma.h", "sk_sync.h", "sk_internal.h"]
# shifted half-pass kernel of each workload (the launch that dominates a solve)
HALF_PASS_KERNEL = {"embed_d64_50k_bf16": "k_lse_mfma<4, 2, true, true, false, false>",
                    "mix8_d3_50k": "k_lse_mfma<2, 2, true, false, true, false>"}


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def kernel_traffic(workload):
    """HBM bytes per launch of the workload's half-pass kernel, or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    k = t.get("kernels", {}).get(HALF_PASS_KERNEL.get(workload, ""))
    if not k:
        return None
    return (k["fetch_kib"] * t["fetch_scale"] + k["write_kib"] * t["write_scale"]) * 1024.0


def _pmc_means(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def summarize_counters(fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """Write TRAFFIC_FILE from four rocprofv3 --pmc output folders and print a summary."""
    fetch, nf = _pmc_means(fetch_dir)
    write, _ = _pmc_means(write_dir)
    cf, _ = _pmc_means(cfetch_dir)
    cw, _ = _pmc_means(cwrite_dir)
    copy_kib = (1 << 30) / 1024.0  # --copy-calibration moves 1 GiB per copy
    name = next(k for k in cf if "copyBuffer" in k)
    fs, ws = copy_kib / cf[name], copy_kib / cw[name]
    kernels = {}
    for full, v in fetch.items():
        for stem in ("k_lse_mfma<", "k_pv_mfma<", "k_lse_gemm<", "k_pv_gemm<"):
            i = full.find(stem)
            if i >= 0:
                short = full[i:full.index(">", i) + 1]
                kernels[short] = {"fetch_kib": v, "write_kib": write.get(full, 0.0), "dispatches": nf[full]}
    out = {"source_digest": source_digest(), "fetch_scale": fs, "write_scale": ws,
           "copy_fetch_kib": cf[name], "copy_write_kib": cw[name], "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    print(f"copy of {copy_kib:.0f} KiB: FETCH_SIZE {cf[name]:.0f} KiB (scale {fs:.3f}), "
          f"WRITE_SIZE {cw[name]:.0f} KiB (scale {ws:.3f})")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB read | scaled MB written |")
    print("|---|---|---|---|---|---|")
    for k, v in sorted(kernels.items()):
        print(f"| `{k}` | {v['dispatches']} | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | "
              f"{v['fetch_kib'] * fs * 1.024e-3:.1f} | {v['write_kib'] * ws * 1.024e-3:.1f} |")


def _dev_points(arr, dtype, torch, dev):
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(arr).to(dev)


class Case:
    def __init__(self, key, torch, sk, dev, k=16, mode=None):
        from dataclasses import replace
        self.w = w = W.CASES[key] if mode is None else replace(W.CASES[key], mode=mode)
        inp = W.make_inputs(w, k=k)
        self.inp = inp
        self.x = _dev_points(inp.x, w.dtype, torch, dev)
        self.y = _dev_points(inp.y, w.dtype, torch, dev)
        self.a = torch.from_numpy(inp.a).to(dev)
        self.b = torch.from_numpy(inp.b).to(dev)
        self.V = torch.from_numpy(inp.V).to(dev)
        self.U = torch.from_numpy(inp.U).to(dev)
        self.k = k
        self.sk = sk
        self.torch = torch
        dt = sk.SK_BF16 if w.dtype == "bf16" else sk.SK_F32
        nbytes = max(sk.workspace_bytes(sk.SK_OP_SOLVE, dt, w.n, w.m, w.d),
                     sk.workspace_bytes(sk.SK_OP_GRAD, dt, w.n, w.m, w.d),
                     sk.workspace_bytes(sk.SK_OP_APPLY, dt, w.n, w.m, w.d, k))
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)

    def step(self, ev=None):
        """One pass of the hot path; with ev, records (start, end) events per call."""
        sk, w, t = self.sk, self.w, self.torch

        def rec():
            if ev is None:
                return None
            e = t.cuda.Event(enable_timing=True)
            e.record()
            return e

        e0 = rec()
        f, g, cost = sk.solve(self.x, self.y, self.a, self.b, w.eps, w.iters, w.mode, workspace=self.ws)
        e1 = rec()
        grad = sk.eot_grad_x(self.x, self.y, self.a, self.b, g, w.eps, workspace=self.ws)
        e2 = rec()
        pv = sk.transport_apply(self.x, self.y, self.a, self.b, f, g, w.eps, self.V, workspace=self.ws)
        e3 = rec()
        ptu = sk.transport_apply(self.x, self.y, self.a, self.b, f, g, w.eps, self.U, transpose=True,
                                 workspace=self.ws)
        e4 = rec()
        if ev is not None:
            ev.append((e0, e1, e2, e3, e4))
        return f, g, cost, grad, pv, ptu

    def overhead_ms(self, reps=5):
        """Duration of a solve with zero iterations (prep and cost only)."""
        t = self.torch
        out = []
        for _ in range(reps):
            s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            s.record()
            self.sk.solve(self.x, self.y, self.a, self.b, self.w.eps, 0, self.w.mode, workspace=self.ws)
            e.record()
            e.synchronize()
            out.append(s.elapsed_time(e))
        return statistics.median(out)


def pass_roofline(w, pass_ms):
    """Roofline of the half-pass kernel. Per pair the VALU must issue one exp2,
    one add (and a multiply for bf16 points); these share the issue port, so
    the ALU roof is VALU_PEAK / slots per pair, or the measured rate of that
    VALU work alone where the chip beats the model. The matrix-core roof is
    the bf16 MFMA peak for the products the pass issues (2d flops per pair for
    bf16 points, 12d for float32 points); the longer ideal time is the bound,
    and the other fraction is reported beside it."""
    r = _pass_roofline(w, pass_ms)
    r["traffic"] = kernel_traffic(w.name)
    return r


def alu_slots_per_pair(w):
    """VALU issue slots one (row, column) pair needs in a half-pass: exp2 at half
    the 64-lane rate (2 slots), the add into the row sum (1) and, for bf16
    points, the multiply by the score scale c2 (1; float32 records carry c2)."""
    return 3 + (1 if w.dtype == "bf16" else 0)


# Measured rates of register-only loops (bench.py --peaks, stored in
# profiles/unit_peaks.json). VALU_PROBE: the half-pass's VALU work per pair
# alone (exp2 + add, or mul + exp2 + add); the chip runs it slightly faster
# than the issue-slot model, so the ALU roof is the larger of the two.
# MIX_PROBE: the same VALU work with the pass's MFMAs interleaved.
UNIT_PEAKS_FILE = os.path.join(ROOT, "profiles", "unit_peaks.json")
VALU_PROBE = {"f32": "exp2_add", "bf16": "mul_exp2_add"}
MIX_PROBE = {("f32", 3): "mix_f32_points_d3", ("bf16", 64): "mix_bf16_points_d64"}


def _unit_peak(name):
    if name is None or not os.path.exists(UNIT_PEAKS_FILE):
        return None
    with open(UNIT_PEAKS_FILE) as fh:
        return json.load(fh)["peaks"].get(name, {}).get("rate")


def measured_mix_rate(w):
    name = MIX_PROBE.get((w.dtype, w.d))
    return name, _unit_peak(name)


def alu_roof(w):
    """(pairs/s, how it was priced): the issue-slot model or, when the chip
    beats it, the measured rate of the same VALU work with nothing else."""
    model = VALU_PEAK / alu_slots_per_pair(w)
    probe = _unit_peak(VALU_PROBE[w.dtype])
    if probe and probe > model:
        return probe, f"measured {VALU_PROBE[w.dtype]} probe ({probe:.4g} pairs/s > model {model:.4g})"
    return model, f"issue-slot model ({alu_slots_per_pair(w)} slots per pair)"


def _pass_roofline(w, pass_ms):
    pairs = w.n * w.m
    sec = pass_ms * 1e-3
    rate = pairs / sec
    alu_peak, alu_basis = alu_roof(w)
    also = {"exp_frac": rate / EXP_PEAK, "alu_roof_basis": alu_basis}
    probe, mix_rate = measured_mix_rate(w)
    if mix_rate:
        also["measured_mix_probe"] = probe
        also["measured_mix_frac"] = rate / mix_rate
    if w.d >= 32:
        # The contraction: 2d flops per pair. bf16 points issue exactly that on
        # the bf16 matrix cores. float32 points issue six bf16 products per
        # coordinate pair (12d flops per pair) for float32 accuracy, so their
        # ceiling is the bf16 peak for that issued work; the fraction of the
        # float32 MFMA peak at 2d flops per pair is kept beside it.
        issued = (2.0 if w.dtype == "bf16" else 12.0) * w.d * pairs
        mfma_frac = issued / sec / BF16_MFMA_PEAK
        if w.dtype != "bf16":
            also["f32_contraction_TFLOPs"] = 2.0 * w.d * pairs / sec / 1e12
            also["f32_contraction_frac_of_f32_mfma_peak"] = 2.0 * w.d * pairs / sec / F32_MFMA_PEAK
        # the binding roof is whichever ideal time is longer
        if issued / BF16_MFMA_PEAK >= pairs / alu_peak:
            also["alu_frac"] = rate / alu_peak
            return {"bound": "mfma", "achieved": issued / sec / 1e12, "peak": BF16_MFMA_PEAK / 1e12,
                    "unit": "TFLOP/s", "frac": mfma_frac, "traffic": None, "also": also}
        also["mfma_frac"] = mfma_frac
        also["mfma_TFLOPs"] = issued / sec / 1e12
    return {"bound": "alu", "achieved": rate / 1e9, "peak": alu_peak / 1e9, "unit": "Gpair/s",
            "frac": rate / alu_peak, "traffic": None, "also": also}


def op_roofline(w, ms, value_width):
    """Roofline of a gradient / application launch (n x m pairs): per pair the
    scores (2d flops) and the weighted sum over the value width (2 * width
    flops) on the matrix cores, and at least the half-pass's exp2 and add on
    the VALU. The longer ideal time is the bound."""
    pairs = w.n * w.m
    sec = ms * 1e-3
    # float32 points issue six bf16 products per coordinate (scores and values)
    peak = BF16_MFMA_PEAK
    flops = (2.0 if w.dtype == "bf16" else 12.0) * (w.d + value_width) * pairs
    alu_peak, _ = alu_roof(w)
    t_mfma, t_alu = flops / peak, pairs / alu_peak
    r = {"ms": ms, "mfma_frac": t_mfma / sec, "alu_frac": t_alu / sec}
    r["bound"] = "mfma" if t_mfma >= t_alu else "alu"
    r["frac"] = max(t_mfma, t_alu) / sec
    return r


def measure(case, steps, warmup):
    torch = case.torch
    for _ in range(warmup):
        case.step()
    torch.cuda.synchronize()
    ov = case.overhead_ms()
    torch.cuda.synchronize()
    ev = []
    t0 = time.perf_counter()
    for _ in range(steps):
        case.step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    solve_ms = [e[0].elapsed_time(e[1]) for e in ev]
    grad_ms = [e[1].elapsed_time(e[2]) for e in ev]
    pv_ms = [e[2].elapsed_time(e[3]) for e in ev]
    ptu_ms = [e[3].elapsed_time(e[4]) for e in ev]
    w = case.w
    pass_ms = (statistics.median(solve_ms) - ov) / (2 * w.iters)
    return {
        "wall_s": wall,
        "ms_per_step": 1e3 * wall / steps,
        "iters_per_s": w.iters * steps / wall,
        "solve_ms_median": statistics.median(solve_ms),
        "solve_ms_q01_q99": [float(np.quantile(solve_ms, 0.01)), float(np.quantile(solve_ms, 0.99))],
        "prep_cost_ms": ov,
        "half_pass_ms": pass_ms,
        "grad_ms": statistics.median(grad_ms),
        "apply_PV_ms": statistics.median(pv_ms),
        "apply_PtU_ms": statistics.median(ptu_ms),
        "solve_only_iters_per_s": w.iters / (statistics.median(solve_ms) * 1e-3),
        "nmd_iters_per_s": w.n * w.m * w.d * w.iters * steps / wall,
        "roofline": pass_roofline(w, pass_ms),
        # every step of the path against its own roof (prep and cost: one
        # zero-iteration solve, O(n + m) work, launch bound)
        "rows": {
            "a1_a6_prep_and_cost_ms": ov,
            "a3_a4_half_pass": {"ms": pass_ms, **{k: v for k, v in pass_roofline(w, pass_ms).items()
                                                  if k in ("bound", "frac")}},
            "a7_grad": op_roofline(w, statistics.median(grad_ms), w.d),
            "a8_PV": op_roofline(w, statistics.median(pv_ms), case.k),
            "a8_PtU": op_roofline(w, statistics.median(ptu_ms), case.k),
        },
    }


def measure_divergence(case, steps, warmup):
    """Debiased divergence S = OT(a,b) - OT(a,a)/2 - OT(b,b)/2 with the gradients
    in a, b, x and y: three solves of `iters` iterations and four gradients per
    evaluation, timed with HIP events on the library's stream."""
    sk, w, torch = case.sk, case.w, case.torch
    dt = sk.SK_BF16 if w.dtype == "bf16" else sk.SK_F32
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_DIVERGENCE, dt, w.n, w.m, w.d) + 256, dtype=torch.uint8,
                     device=case.x.device)
    for _ in range(warmup):
        sk.sinkhorn_divergence(case.x, case.y, case.a, case.b, w.eps, w.iters, w.mode, workspace=ws)
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        S, *_ = sk.sinkhorn_divergence(case.x, case.y, case.a, case.b, w.eps, w.iters, w.mode, workspace=ws)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = statistics.median(ms)
    return {"metric": "debiased Sinkhorn divergence evaluations/s (with gradients in a, b, x, y)",
            "value": 1e3 / med, "unit": "evaluations/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_eval": med, "higher_is_better": True, "dtype": "bf16" if w.dtype == "bf16" else "f32",
            "data": "synthetic", "divergence": float(S),
            "config": {"workload": w.name, "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "iters": w.iters,
                       "mode": w.mode, "evaluation": "3 solves (n x m, n x n, m x m) + 4 gradients"},
            "solve_iters_per_s": 3 * w.iters / (med * 1e-3)}


def measure_hvp(case, steps, warmup):
    """Hessian-vector products of OT_eps in x at the workload's solved pair
    (CG to a relative residual of 1e-6), timed on the host (the call blocks)."""
    sk, w, torch = case.sk, case.w, case.torch
    f, g, _ = sk.solve(case.x, case.y, case.a, case.b, w.eps, w.iters, w.mode, workspace=case.ws)
    dt = sk.SK_BF16 if w.dtype == "bf16" else sk.SK_F32
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_HVP, dt, w.n, w.m, w.d) + 256, dtype=torch.uint8,
                     device=case.x.device)
    gen = torch.Generator(device=case.x.device).manual_seed(11)
    V = torch.randn(w.n, w.d, generator=gen, device=case.x.device)
    for _ in range(warmup):
        sk.ot_hvp_x(case.x, case.y, case.a, case.b, f, g, w.eps, V, workspace=ws)
    torch.cuda.synchronize()
    sec, its = [], 0
    for _ in range(steps):
        t0 = time.perf_counter()
        _, its, resid = sk.ot_hvp_x(case.x, case.y, case.a, case.b, f, g, w.eps, V, workspace=ws)
        torch.cuda.synchronize()
        sec.append(time.perf_counter() - t0)
    med = statistics.median(sec)
    return {"metric": "Hessian-vector products/s of OT_eps in x", "value": 1.0 / med, "unit": "HVP/s",
            "seconds_per_hvp": med, "cg_iters": its, "cg_residual": resid, "higher_is_better": True,
            "n_gpus": 1, "data": "synthetic", "steps": steps, "warmup": warmup,
            "config": {"workload": w.name, "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "cg_tol": 1e-6}}


def measure_newton(case, steps, sk_tol=1e-4):
    """Newton-CG on the workload's x (float32 points): wall time, costs and
    gradient norms of `steps` steps (blocking)."""
    sk, w, torch = case.sk, case.w, case.torch
    sk.ot_newton_x(case.x, case.y, case.a, case.b, w.eps, newton_iters=1, sk_tol=sk_tol, sk_max_iters=5000)
    torch.cuda.synchronize()
    print("[newton] warm-up done", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    _, costs, norms, done = sk.ot_newton_x(case.x, case.y, case.a, case.b, w.eps, newton_iters=steps,
                                           sk_tol=sk_tol, sk_max_iters=5000)
    sec = time.perf_counter() - t0
    return {"metric": "Newton-CG steps/s on x -> OT_eps(mu_x, nu)", "value": done / sec if done else 0.0,
            "unit": "steps/s", "seconds": sec, "steps": done, "costs": costs, "grad_norms": norms,
            "higher_is_better": True, "n_gpus": 1, "data": "synthetic",
            "config": {"workload": w.name, "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "sk_tol": sk_tol}}


def measure_tol(case, tol, check_every=10, max_iters=20000, eps_start=0.0):
    """Iterations and wall time to reach a marginal error of tol (blocking solve
    with a check every `check_every` iterations)."""
    sk, w, torch = case.sk, case.w, case.torch
    dt = sk.SK_BF16 if w.dtype == "bf16" else sk.SK_F32
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_SOLVE_TOL, dt, w.n, w.m, w.d) + 256, dtype=torch.uint8,
                     device=case.x.device)
    sk.solve_tol(case.x, case.y, case.a, case.b, w.eps, tol, 20, w.mode, check_every, workspace=ws)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, _, cost, done, err = sk.solve_tol(case.x, case.y, case.a, case.b, w.eps, tol, max_iters, w.mode,
                                         check_every, eps_start=eps_start, workspace=ws)
    sec = time.perf_counter() - t0
    return {"metric": "iterations to a marginal error of tol", "value": done, "unit": "iterations",
            "higher_is_better": False, "seconds": sec, "iters_per_s": done / sec, "err": err, "tol": tol,
            "converged": err <= tol, "cost": float(cost), "check_every": check_every, "max_iters": max_iters,
            "eps_start": eps_start,
            "n_gpus": 1, "data": "synthetic",
            "config": {"workload": w.name, "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "mode": w.mode}}


def io_model(w, tile):
    """Algorithmic operand bytes a GEMM-tiled half-pass moves into the CUs
    with an R x C workgroup tile: every (row block, column block) pair reads
    both blocks' records once, n m s (1/C + 1/R) bytes for s bytes a record
    (IO bound of the pass: review, Summary, Theorem 2's n m d^2 / M term, M
    ~ R + C records staged)."""
    R, C = tile
    s = (w.d if w.dtype == "bf16" else 6 * w.d) * 2  # bf16 slots of a record
    s = -(-s // 128) * 128                           # whole 128-byte K chunks
    return w.n * w.m * s * (1.0 / C + 1.0 / R)


GEMM_TILES = {"256x256": (256, 256), "128x128": (128, 128), "128x256": (128, 256)}


def measure_io_tile(case, reps=5):
    """Shifted half-pass time at the tile FLASHSK_GEMM_TILE selects (large-d workloads)."""
    sk, w, torch = case.sk, case.w, case.torch
    tile = os.environ.get("FLASHSK_GEMM_TILE", "256x256")
    if tile not in GEMM_TILES:
        raise SystemExit(f"FLASHSK_GEMM_TILE={tile}: not one of {sorted(GEMM_TILES)}")

    def run(iters):
        out = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            sk.solve(case.x, case.y, case.a, case.b, w.eps, iters, "alternating", workspace=case.ws)
            e.record()
            e.synchronize()
            out.append(s.elapsed_time(e))
        return statistics.median(out)

    run(2)
    ms = (run(11) - run(1)) / 20.0
    model = io_model(w, GEMM_TILES[tile])
    return {"metric": "shifted half-pass time", "value": ms, "unit": "ms", "higher_is_better": False,
            "tile": tile, "model_operand_bytes": model, "model_operand_TBps": model / (ms * 1e-3) / 1e12,
            "config": {"workload": w.name, "n": w.n, "m": w.m, "d": w.d, "dtype": w.dtype}}


def summarize_io(pairs):
    """Markdown table of the re-read study from TILE=TIMING_JSON:FETCH_DIR:REQ_DIR triples."""
    print("| tile | half-pass ms | model operand MB (n m s (1/R + 1/C)) | L2 requests (TCC_REQ) x 128 B, MB "
          "| L2 hit rate | FETCH_SIZE MB (x copy scale) |")
    print("|---|---|---|---|---|---|")
    try:
        with open(TRAFFIC_FILE) as fh:
            fscale = json.load(fh)["fetch_scale"]
    except (OSError, ValueError, KeyError):
        fscale = 1.0
    for item in pairs:
        tile, rest = item.split("=", 1)
        tfile, fdir, rdir = rest.split(":")
        with open(tfile) as fh:
            t = json.loads(fh.read().strip().splitlines()[-1])
        fetch, _ = _pmc_means(fdir)
        req, _ = _pmc_means(rdir)
        stem = "k_lse_gemm<true"
        kf = next(v for k, v in fetch.items() if stem in k)
        # TCC_REQ and TCC_HIT arrive as separate counter rows: take both by name
        import csv
        import glob
        vals = {}
        for f in glob.glob(os.path.join(rdir, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if stem in r["Kernel_Name"]:
                        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        reqs = sum(vals["TCC_REQ_sum"]) / len(vals["TCC_REQ_sum"])
        hits = sum(vals["TCC_HIT_sum"]) / len(vals["TCC_HIT_sum"])
        print(f"| {tile} | {t['value']:.3f} | {t['model_operand_bytes'] / 1e6:.0f} | {reqs * 128 / 1e6:.0f} | "
              f"{hits / reqs:.2f} | {kf * fscale * 1.024e-3:.0f} |")


def measure_low_eps(case, eps_list=(1e-2, 3e-3, 1e-3, 3e-4), tols=(1e-3, 1e-4, 1e-5), eps_start=1.0,
                    check_every=10, max_iters=20000):
    """Iterations and time to a marginal tolerance on the workload's points at
    each eps, with and without eps-scaling (one iteration per halving from
    eps_start), in the workload's schedule; each run blocks on its checks."""
    from dataclasses import replace
    sk, torch = case.sk, case.torch
    dt = sk.SK_BF16 if case.w.dtype == "bf16" else sk.SK_F32
    w0 = case.w
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_SOLVE_TOL, dt, w0.n, w0.m, w0.d) + 256, dtype=torch.uint8,
                     device=case.x.device)
    sk.solve_tol(case.x, case.y, case.a, case.b, w0.eps, 1e-3, 20, w0.mode, check_every, workspace=ws)  # warm-up
    rows = []
    for eps in eps_list:
        w = replace(w0, eps=eps)
        for es in (0.0, eps_start):
            for tol in tols:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                f, _, cost, done, err = sk.solve_tol(case.x, case.y, case.a, case.b, eps, tol, max_iters, w.mode,
                                                     check_every, eps_start=es, workspace=ws)
                sec = time.perf_counter() - t0
                floor = 2.0 ** -24 * float(f.abs().max()) / eps
                rows.append({"eps": eps, "eps_start": es, "tol": tol, "iters": done, "converged": err <= tol,
                             "err": err, "seconds": sec, "iters_per_s": done / sec, "cost": float(cost),
                             "f32_floor_estimate": floor})
                print(f"[low-eps] eps={eps:g} eps_start={es:g} tol={tol:g}: {done} iterations, err {err:.3e}, "
                      f"{sec:.3f} s, floor ~{floor:.1e}", file=sys.stderr, flush=True)
    return {"metric": "iterations to a marginal error of tol at low eps", "unit": "iterations",
            "higher_is_better": False, "n_gpus": 1, "data": "synthetic", "check_every": check_every,
            "max_iters": max_iters,
            "config": {"workload": w0.name, "n": w0.n, "m": w0.m, "d": w0.d, "mode": w0.mode},
            "rows": rows}


def measure_hadamard(case, r, steps, warmup):
    """(P o A B^T) V and (P o A B^T)^T U with the workload's potentials (one
    solve first) and k = 16: ceil(r / 4) matrix-free applications each."""
    sk, w, torch = case.sk, case.w, case.torch
    f, g, _ = sk.solve(case.x, case.y, case.a, case.b, w.eps, w.iters, w.mode, workspace=case.ws)
    gen = torch.Generator(device=case.x.device).manual_seed(7)
    A = torch.randn(w.n, r, generator=gen, device=case.x.device)
    B = torch.randn(w.m, r, generator=gen, device=case.x.device)
    dt = sk.SK_BF16 if w.dtype == "bf16" else sk.SK_F32
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_APPLY_HADAMARD, dt, w.n, w.m, w.d, case.k) + 256,
                     dtype=torch.uint8, device=case.x.device)

    def run():
        sk.transport_apply_hadamard(case.x, case.y, case.a, case.b, f, g, w.eps, A, B, case.V, workspace=ws)
        sk.transport_apply_hadamard(case.x, case.y, case.a, case.b, f, g, w.eps, A, B, case.U, transpose=True,
                                    workspace=ws)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = statistics.median(ms)
    return {"metric": "Hadamard-weighted applications/s ((P o W) V and (P o W)^T U, W = A B^T)",
            "value": 2e3 / med, "unit": "applications/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_pair_of_applications": med, "higher_is_better": True,
            "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
            "config": {"workload": w.name, "n": w.n, "m": w.m, "d": w.d, "eps": w.eps, "rank": r, "k": case.k,
                       "applications_per_call": -(-r // max(1, 64 // case.k))}}


def cpu_baseline(case, target_s=15.0):
    """The float64 oracle on the host cores, on a bounded sample of the workload:
    the F map on R rows of x and the G map on R rows of y (all columns each),
    scaled to one full iteration (n rows of F, m rows of G); when a whole
    iteration takes less than the target, whole iterations are repeated."""
    import oracle

    oracle.build(force=False)
    w, inp = case.w, case.inp
    x64, y64 = inp.x64(), inp.y64()
    g = np.zeros(w.m)
    f = np.zeros(w.n)
    lim = min(w.n, w.m)
    r0, t0 = 16, 0.0
    while True:  # ramp up until the fixed costs are small against the sample
        t = time.perf_counter()
        oracle.F(x64[:r0], y64, inp.b, g, w.eps)
        oracle.G(x64, y64[:r0], inp.a, f, w.eps)
        t0 = time.perf_counter() - t
        if t0 >= 0.1 * target_s or r0 >= lim:
            break
        r0 = min(lim, r0 * 8)
    per_row = t0 / (2 * r0)
    R = int(max(16, min(lim, target_s / (2 * per_row))))
    reps = 1
    if R >= min(w.n, w.m):
        R = min(w.n, w.m)
        reps = max(1, int(round(target_s / (per_row * (w.n + w.m)))))
    tf = tg = 0.0
    for _ in range(reps):
        t = time.perf_counter()
        oracle.F(x64[:R], y64, inp.b, g, w.eps)
        tf += time.perf_counter() - t
        t = time.perf_counter()
        oracle.G(x64, y64[:R], inp.a, f, w.eps)
        tg += time.perf_counter() - t
    sec_per_iter = (tf * w.n / R + tg * w.m / R) / reps
    return {"value": 1.0 / sec_per_iter, "unit": "iters/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"F map on {R} rows of x and G map on {R} rows of y (all {w.m} and {w.n} columns), "
                      f"float64, {reps} time(s), scaled by n/{R} and m/{R} to one iteration; "
                      f"{tf + tg:.1f} s measured"}


def cpu_single_thread_tiny(min_s=2.0):
    """Scaling context for the CPU baseline: the float64 oracle on one host
    thread, whole iterations of the tiny configuration (n = m = 1024, d = 3)."""
    import oracle

    oracle.build(force=False)
    w = W.CASES[1]
    inp = W.make_inputs(w)
    x64, y64 = inp.x64(), inp.y64()
    before = oracle.threads()
    oracle.set_threads(1)
    try:
        its, t0 = 0, time.perf_counter()
        while True:
            oracle.solve(x64, y64, inp.a, inp.b, w.eps, 1, w.mode)
            its += 1
            sec = time.perf_counter() - t0
            if sec >= min_s:
                break
    finally:
        oracle.set_threads(before)
    return {"value": its / sec, "unit": "iters/s", "cores": 1, "kind": "oracle",
            "sample": f"{its} whole iteration(s) of {w.name} (n=m={w.n}, d={w.d}) on one thread, {sec:.1f} s"}


# Unit-rate microbenchmarks (streaming_sinkhorn_solver_log_amd/peaks/peaks.hip):
# (index, name, unit of the work count, model peak per second or None, model)
PEAK_CASES = [
    (0, "exp2", "exp/s", EXP_PEAK, "v_exp_f32 at 2 issue slots"),
    (1, "fma_f32", "op/s", VALU_PEAK, "non-packed fp32 VALU, 1 slot"),
    (2, "add_f32", "op/s", VALU_PEAK, "non-packed fp32 VALU, 1 slot"),
    (3, "exp2_add", "score/s", VALU_PEAK / 3, "exp2 (2 slots) + add (1 slot) per score"),
    (4, "mfma_bf16_32x32x16", "flop/s", BF16_MFMA_PEAK, "published dense bf16"),
    (5, "mfma_f32_32x32x2", "flop/s", F32_MFMA_PEAK, "published fp32 matrix"),
    (6, "mix_f32_points_d3", "score/s", VALU_PEAK / 3,
     "2 bf16 MFMAs per 1024 scores + exp2 + add: VALU roof if the MFMAs hide fully"),
    (7, "hbm_read", "B/s", HBM_PEAK, "published HBM3E"),
    (8, "l2_read", "B/s", None, "1 MiB read by every workgroup"),
    (9, "mall_read", "B/s", None, "64 MiB streamed 32 times"),
    (10, "mix_bf16_points_d64", "score/s", VALU_PEAK / 4,
     "4 bf16 MFMAs per 1024 scores + mul + exp2 + add: VALU roof if the MFMAs hide fully"),
    (11, "mul_exp2_add", "score/s", VALU_PEAK / 4, "mul + exp2 (2 slots) + add per score"),
]


def measure_peaks(wgs_list=None):
    """Unit-rate microbenchmarks at 8 workgroups per CU; with wgs_list, the
    half-pass mix probes and their parts at each of those workgroup counts."""
    import ctypes

    from streaming_sinkhorn_solver_log_amd.build import PEAKS_LIB
    if not os.path.exists(PEAKS_LIB):
        raise RuntimeError(f"{PEAKS_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.skp_measure.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    lib.skp_measure.restype = ctypes.c_int
    res = {}
    cus = ctypes.c_int(0)

    def run(which, name, wgs):
        work, ms = ctypes.c_double(0), ctypes.c_double(0)
        rc = lib.skp_measure(which, wgs, ctypes.byref(work), ctypes.byref(ms), ctypes.byref(cus))
        if rc != 0:
            raise RuntimeError(f"peaks benchmark {name} failed with code {rc}")
        return work.value / (ms.value * 1e-3), ms.value

    if wgs_list:
        for which, name, unit, peak, model in PEAK_CASES:
            if which not in (3, 4, 6, 10, 11):
                continue
            res[name] = {"unit": unit, "by_wgs_per_cu": {}}
            for wgs in wgs_list:
                rate, ms = run(which, name, wgs)
                res[name]["by_wgs_per_cu"][str(wgs)] = {"rate": rate, "ms": ms}
                print(f"[peaks] {name} at {wgs} workgroups/CU: {rate:.4g} {unit} ({ms:.3f} ms)",
                      file=sys.stderr, flush=True)
        return {"peaks_by_occupancy": res, "cus": cus.value}
    for which, name, unit, peak, model in PEAK_CASES:
        rate, ms = run(which, name, 0)
        res[name] = {"rate": rate, "unit": unit, "ms": ms, "model_peak": peak,
                     "frac": rate / peak if peak else None, "model": model,
                     "per_cu_per_clk": rate / (CU * CLK)}
        print(f"[peaks] {name}: {rate:.4g} {unit} ({ms:.3f} ms)", file=sys.stderr, flush=True)
    return {"peaks": res, "cus": cus.value, "clock_assumed_hz": CLK}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="embed_d64_50k_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--no-d3", action="store_true", help="skip the d=3 point")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--divergence", action="store_true",
                    help="time the debiased Sinkhorn divergence with its four gradients instead of the step")
    ap.add_argument("--hadamard", type=int, default=0, metavar="R",
                    help="time the Hadamard-weighted applications (P o A B^T) V and their transposes, rank R")
    ap.add_argument("--tol", type=float, default=0.0,
                    help="solve the workload to this marginal error (checked every 10 iterations, at most "
                         "20000) and report the iterations and time it took")
    ap.add_argument("--eps-start", type=float, default=0.0,
                    help="with --tol: eps-scaling from this eps (one iteration per halving)")
    ap.add_argument("--low-eps-study", action="store_true",
                    help="iterations and time to marginal tolerances 1e-3..1e-5 at eps 1e-2..3e-4, with and "
                         "without eps-scaling, on the workload's points")
    ap.add_argument("--newton", type=int, default=0, metavar="K",
                    help="time K steps of Newton-CG on the workload's x (float32 points)")
    ap.add_argument("--hvp", action="store_true",
                    help="time one Hessian-vector product of OT_eps in x at the workload's solved pair")
    ap.add_argument("--peaks", action="store_true",
                    help="only run the unit-rate microbenchmarks (exp2, VALU, MFMA, HBM/L2/MALL reads)")
    ap.add_argument("--peaks-wgs", default="", metavar="N,N,...",
                    help="with --peaks: run the half-pass mix probes at these workgroups per CU instead")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy (scale for the HBM counters)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/hbm_traffic.json from four rocprofv3 --pmc output folders")
    ap.add_argument("--io-study", action="store_true",
                    help="time the shifted GEMM-tiled half-pass at the tile FLASHSK_GEMM_TILE selects "
                         "(256x256, 128x128, 128x256) and print it with the re-read model")
    ap.add_argument("--summarize-io", nargs="+", metavar="TILE=TIMING:FETCH_DIR:REQ_DIR",
                    help="print the re-read study table from timing JSON files and rocprofv3 --pmc folders "
                         "(FETCH_SIZE; TCC_REQ_sum TCC_HIT_sum)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_io:
        summarize_io(args.summarize_io)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import streaming_sinkhorn_solver_log_amd as sk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.peaks:
        wgs = [int(v) for v in args.peaks_wgs.split(",") if v.strip()]
        print(json.dumps(measure_peaks(wgs)), flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "copies": 3}), flush=True)
        return
    key = WORKLOADS[args.workload]
    print(f"[bench] workload {args.workload}: building inputs", file=sys.stderr, flush=True)
    case = Case(key, torch, sk, dev)
    if args.io_study:
        print(json.dumps(measure_io_tile(case)), flush=True)
        return
    if args.divergence:
        print(json.dumps(measure_divergence(case, args.steps, args.warmup)), flush=True)
        return
    if args.hvp:
        print(json.dumps(measure_hvp(case, args.steps, args.warmup)), flush=True)
        return
    if args.newton:
        print(json.dumps(measure_newton(case, args.newton)), flush=True)
        return
    if args.low_eps_study:
        print(json.dumps(measure_low_eps(case)), flush=True)
        return
    if args.tol > 0:
        print(json.dumps(measure_tol(case, args.tol, eps_start=args.eps_start)), flush=True)
        return
    if args.hadamard:
        print(json.dumps(measure_hadamard(case, args.hadamard, args.steps, args.warmup)), flush=True)
        return
    print(f"[bench] timing {args.steps} steps after {args.warmup} warm-up", file=sys.stderr, flush=True)
    r = measure(case, args.steps, args.warmup)
    w = case.w
    out = {
        "metric": METRIC,
        "value": r["iters_per_s"],
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "m": w.m, "d": w.d, "point_dtype": w.dtype,
                   "eps": w.eps, "iters": w.iters, "mode": w.mode, "weights": w.weights,
                   "step": f"solve({w.iters} iters) + eot_grad_x + P.V + P^T.U (k=16)"},
        "roofline": r["roofline"],
        "detail": {k: v for k, v in r.items() if k != "roofline"},
    }
    if not args.no_d3 and key != 6:
        print("[bench] d=3 point", file=sys.stderr, flush=True)
        c3 = Case(6, torch, sk, dev)
        r3 = measure(c3, args.steps, args.warmup)
        out["d3"] = {"workload": c3.w.name, "iters_per_s": r3["iters_per_s"], "ms_per_step": r3["ms_per_step"],
                     "roofline": r3["roofline"], "detail": {k: v for k, v in r3.items() if k != "roofline"}}
        del c3
        # the same shape in the averaged schedule: both half-passes in one launch
        print("[bench] d=3 point, symmetric schedule", file=sys.stderr, flush=True)
        c3s = Case(6, torch, sk, dev, mode="symmetric")
        r3s = measure(c3s, args.steps, args.warmup)
        out["d3"]["symmetric"] = {"iters_per_s": r3s["iters_per_s"], "ms_per_step": r3s["ms_per_step"],
                                  "solve_only_iters_per_s": r3s["solve_only_iters_per_s"],
                                  "half_pass_ms": r3s["half_pass_ms"],
                                  "half_pass_frac": r3s["roofline"]["frac"]}
        del c3s
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        out["cpu_baseline"]["single_thread_tiny"] = cpu_single_thread_tiny()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
