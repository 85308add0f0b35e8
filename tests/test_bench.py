"""Host-side logic of bench.py: the single-GPU rule, the roofline accounting of
the half-pass and of the gradient / application launches, and the HBM traffic
lookup (no GPU needed)."""
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_half_pass_roofline_bf16_d64_is_alu_bound():
    w = W.CASES[3]  # n = m = 50k, d = 64, bf16
    ms = 0.4
    r = bench._pass_roofline(w, ms)
    pairs = w.n * w.m
    model = bench.VALU_PEAK / 4  # exp2 (2 slots) + add + multiply by c2
    alu_peak, basis = bench.alu_roof(w)
    assert alu_peak >= model  # never a roof the chip already beats
    probe = bench._unit_peak("mul_exp2_add")
    if probe:
        assert alu_peak == pytest.approx(max(model, probe))
    assert r["bound"] == "alu" and r["unit"] == "Gpair/s"
    assert r["frac"] == pytest.approx(pairs / (ms * 1e-3) / alu_peak)
    assert r["achieved"] == pytest.approx(pairs / (ms * 1e-3) / 1e9)
    assert r["also"]["alu_roof_basis"] == basis
    # the matrix-core ideal (2d flops per pair at the bf16 peak) is the shorter one, reported beside
    assert r["also"]["mfma_frac"] == pytest.approx(2 * w.d * pairs / (ms * 1e-3) / bench.BF16_MFMA_PEAK)
    assert r["also"]["mfma_frac"] < r["frac"]


def test_half_pass_roofline_float32_d3_counts_three_slots():
    w = W.CASES[6]  # n = m = 50k, d = 3, float32 records carry the score scale
    r = bench._pass_roofline(w, 0.25)
    assert r["bound"] == "alu"
    assert r["peak"] >= bench.VALU_PEAK / 3 / 1e9
    assert r["peak"] == pytest.approx(bench.alu_roof(w)[0] / 1e9)
    assert "mfma_frac" not in r["also"]  # d < 32: no matrix-core roof


def test_half_pass_roofline_float32_large_d_is_priced_at_the_issued_bf16_work():
    w = W.CASES[4]  # n = m = 20k, d = 512, float32: six bf16 products per coordinate
    ms = 2.5
    r = bench._pass_roofline(w, ms)
    pairs = w.n * w.m
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["peak"] == pytest.approx(bench.BF16_MFMA_PEAK / 1e12)
    assert r["frac"] == pytest.approx(12 * w.d * pairs / (ms * 1e-3) / bench.BF16_MFMA_PEAK)
    assert r["frac"] <= 1.0
    # the float32 contraction's own fraction is kept beside it
    assert r["also"]["f32_contraction_frac_of_f32_mfma_peak"] == pytest.approx(
        2 * w.d * pairs / (ms * 1e-3) / bench.F32_MFMA_PEAK)


def test_op_roofline_takes_the_longer_ideal():
    w = W.CASES[3]
    r = bench.op_roofline(w, 1.5, 64)
    assert r["frac"] == pytest.approx(max(r["mfma_frac"], r["alu_frac"]))
    assert r["bound"] == ("mfma" if r["mfma_frac"] >= r["alu_frac"] else "alu")


def test_traffic_is_reported_only_for_the_counted_kernel_sources():
    for name in ("embed_d64_50k_bf16", "mix8_d3_50k"):
        t = bench.kernel_traffic(name)
        if t is None:
            pytest.skip("the half-pass sources changed since the HBM counters were taken")
        # the records of both sides alone are read once: at least 2 x n x record bytes
        w = W.CASES[{"embed_d64_50k_bf16": 3, "mix8_d3_50k": 6}[name]]
        assert t > 2 * w.n * 32
    assert bench.kernel_traffic("no_such_workload") is None
