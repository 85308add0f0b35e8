"""The seeded input generators: determinism, storage rounding, shapes."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_is_round_to_nearest_even():
    one = np.float32(1.0)
    vals = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -2.5, 3.0e-39], dtype=np.float32)
    bits = W.f32_to_bf16_bits(vals)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80          # halfway, ties to the even neighbour 1.0
    assert bits[2] == 0x3F82          # halfway, ties to the even neighbour 1.015625
    assert W.bf16_bits_to_f32(bits[:1])[0] == one
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100_000) * 10.0 ** rng.uniform(-5, 5, 100_000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), ref)
    back = W.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("key", sorted(W.CASES))
def test_inputs_are_deterministic_and_shaped(key):
    w = W.CASES[key].scaled(257, 131)
    i1, i2 = W.make_inputs(w), W.make_inputs(w)
    for a1, a2 in [(i1.x, i2.x), (i1.y, i2.y), (i1.a, i2.a), (i1.b, i2.b)]:
        assert a1.tobytes() == a2.tobytes()
    assert i1.x.shape == (257, w.d) and i1.y.shape == (131, w.d)
    assert i1.x.dtype == (np.uint16 if w.dtype == "bf16" else np.float32)
    assert i1.a.dtype == np.float32 and i1.b.dtype == np.float32
    assert np.all(i1.a > 0) and np.all(i1.b > 0)
    assert abs(float(i1.a.astype(np.float64).sum()) - 1.0) < 1e-5
    if w.apply_k:
        assert i1.V.shape == (131, w.apply_k) and i1.U.shape == (257, w.apply_k)
    assert np.all(np.isfinite(i1.x64())) and np.all(np.isfinite(i1.y64()))


def test_bf16_variant_shares_points_with_f32_config():
    a = W.make_inputs(W.CASES[4].scaled(64))
    b = W.make_inputs(W.CASES[7].scaled(64))
    assert np.array_equal(W.f32_to_bf16_bits(a.x), b.x)
